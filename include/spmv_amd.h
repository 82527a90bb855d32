/*
 * spmv_amd.h -- C ABI of the MI355X sparse matrix-vector library.
 *
 * The library computes y = alpha * A * x + beta * y for a large, very sparse
 * general square matrix A held on one GPU in one of five storage formats:
 *
 *   CSR       compressed sparse rows (row pointer, column, value), the input
 *             form and the canonical copy ("Development of Krylov and AMG
 *             linear solvers for large-scale sparse matrices on GPUs",
 *             Sect. 2.1, Fig. 3: Ap holds the start of each row, Aj and Ax
 *             the columns and values).
 *   ELLPACK-R rows shifted left into an n x Nmax rectangle stored column by
 *             column, the row count padded to a multiple of the SIMD width
 *             (64 on gfx950), plus the length of every row so that work
 *             stops at the row's end ("Sparse matrix-vector multiplication
 *             on GPGPU clusters", Sect. 2.1, Fig. 1, footnote 2, Fig. 2b).
 *             Each slot keeps its value and column side by side (one
 *             record), so a slot read on its own costs one cache line.
 *   SELL-64   the pJDS idea of the same page (Sect. 2.2): rows sorted by
 *             length, longest first, cut into blocks of 64 rows each padded
 *             to its longest row, stored block by block, with the row
 *             permutation.  apply() works in the caller's row order.
 *   HYB       an ELL part of width K plus the remaining entries of every row
 *             in coordinate (row, col, val) form ("Development of Krylov...",
 *             Sect. 2.1, Fig. 2; "Load-balancing Sparse Matrix Vector
 *             Product Kernels on GPUs", abstract).
 *   HEC       an ELL part of width K plus the remaining entries in CSR form
 *             ("Development of Krylov...", Sect. 2.1, Fig. 3); the ELL part
 *             is applied first, then the irregular part.  The ELL part of
 *             HYB and HEC is stored column by column in blocks of 1024 rows
 *             (the same page sets the ELL stride to 256 or a multiple of it,
 *             rather than to the matrix height).
 *
 * Conventions shared by all entry points
 *   - Every array argument is a DEVICE pointer (e.g. a torch tensor's
 *     data_ptr()), never a host pointer.  Host pointers appear only in
 *     spmv_export (destination buffer) and in the out-parameters.
 *   - Indices are 0-based.  Rows and columns lie in [0, n).  n < 2^31 - 1
 *     and nnz <= 2^31 - 65537 (the kernels' 32-bit entry indices keep that
 *     headroom).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Functions return 0 (SPMV_OK) or a negative spmv_status; nothing is
 *     thrown across the ABI.  After a non-zero return spmv_last_error()
 *     holds a message for the calling thread.  Kernel faults inside
 *     spmv_apply surface at the caller's next synchronisation, since apply
 *     is asynchronous.
 *   - A handle may be used by several threads for spmv_apply at once (on
 *     different streams), whatever its format and kernels: an apply writes
 *     only y and keeps no buffer of its own.  spmv_convert / spmv_destroy
 *     must not overlap any other call on the same handle.
 */
#ifndef SPMV_AMD_H
#define SPMV_AMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spmv_handle *spmv_t;

/* value type */
typedef enum { SPMV_F32 = 1, SPMV_F64 = 2 } spmv_dtype;

/* storage formats */
typedef enum {
    SPMV_CSR = 0,
    SPMV_ELLR = 1,
    SPMV_SELL64 = 2,
    SPMV_HYB = 3,
    SPMV_HEC = 4,
    /* spmv_convert only: build every eligible format in turn with the given
     * options, time one apply of each on the device and keep the fastest
     * (spmv_info then reports the format kept).  ELL-R is eligible while its
     * padded slots are at most 1.5 times the stored entries; a format over
     * the footprint budget is skipped.  The choice from the row-length
     * statistics that "Load-balancing Sparse Matrix Vector Product Kernels
     * on GPUs" (abstract) and "Development of Krylov...", Sect. 4, make per
     * matrix is made here by measurement. */
    SPMV_AUTO = 5
} spmv_format;

/* CSR apply kernels (spmv_convert_opts.csr_kernel, spmv_info_t.csr_kernel);
 * for HEC the same option picks the kernel of the CSR tail
 * (spmv_info_t.tail_kernel) */
typedef enum {
    SPMV_CSR_AUTO = 0,     /* time the kernels on the device, keep the faster */
    SPMV_CSR_VECTOR = 1,   /* a group of lanes per row (subwave, csr_rows) */
    SPMV_CSR_BALANCED = 2, /* the same number of entries per wave, whatever
                              the row lengths ("Load-balancing Sparse Matrix
                              Vector Product Kernels on GPUs", abstract: a
                              CSR kernel for unbalanced matrices) */
    SPMV_CSR_XBLOCK = 3    /* CSR format, and the tails of HYB and HEC
                              (each range's sum added onto the ELL part's
                              y, from a copy of the tail): the columns cut
                              into 8 slices and the rows into ranges of
                              about equal entry counts (at most 20,480 rows
                              in fp64, 40,960 in fp32); one workgroup sums
                              a range in LDS, slice by slice, starting with
                              the slice of its XCD, so each XCD's x reads
                              stay in its L2
                              ("Sparse matrix-vector multiplication on GPGPU
                              clusters", Sect. 2.3, right-hand-side reuse),
                              then writes the range's y once.  When most
                              entries lie near the diagonal, those within
                              55,296 (fp64) or 12,288 (fp32) columns of
                              their range form a ninth tile, summed last,
                              whose column and row offset share 4 bytes.
                              Stores a second copy of the entries, by tile
                              and by column inside a tile, with 2-byte row
                              offsets outside the band tile; needs 9 n <
                              2^31 - 16.  SPMV_CSR_AUTO times it
                              as well when x is over 4 MiB and the copy fits
                              the footprint budget, and keeps it only when
                              clearly faster. */
} spmv_csr_kernel;

/* input layout of spmv_create */
typedef enum { SPMV_IN_CSR = 0, SPMV_IN_COO = 1 } spmv_input;

/* return codes */
typedef enum {
    SPMV_OK = 0,
    SPMV_ERR_INVALID_ARG = -1,    /* null pointer, bad size or enum, x/y overlap */
    SPMV_ERR_INVALID_MATRIX = -2, /* rowptr not monotone / rowptr[0] != 0 /
                                     rowptr[n] != nnz / index outside [0, n) */
    SPMV_ERR_NO_MEMORY = -3,      /* a device allocation failed */
    SPMV_ERR_FOOTPRINT = -4,      /* padded format larger than the budget */
    SPMV_ERR_HIP = -5,            /* HIP runtime error (message has details) */
    SPMV_ERR_STATE = -6           /* null handle, or array not present */
} spmv_status;

/* options of spmv_convert (pass NULL for all defaults) */
typedef struct {
    /* HYB/HEC: width K of the ELL part.  -1 picks
     * K = max{k >= 0 : #{rows with length >= k} >= ceil(n/3)};
     * a value >= 0 is used as given, clamped to the longest row. */
    int32_t ell_width;
    /* CSR: lanes cooperating on one row, a power of two in 1..64.  0 times
     * every candidate (and 1, 2 or 4 rows per lane group) on the device
     * during the conversion and keeps the fastest; a fixed value only
     * chooses the rows per group.  (The subwarp rule of "Sparse Linear
     * Algebra on AMD and NVIDIA GPUs -- The Race Is On" -- threads per row
     * follow the maximum row length -- is the value spmv_create starts
     * with.) */
    int32_t subwave;
    /* ELL-R / SELL-64 / HYB / HEC / balanced CSR: stage x in LDS.  The
     * workgroup keeps the x entries within about +-9,700 (fp64) or +-19,900
     * (fp32) positions of its rows in a window that slides with the rows
     * (the banded structure of FEM and stencil matrices); entries outside
     * the window are read from global memory.  -1 decides from the matrix:
     * a candidate when at least half of the entries fall inside the window
     * (for ELL-R only when the longest row has at most 128 entries), then
     * one apply with and one without it are timed and the window is kept
     * when clearly faster; 0 off, 1 on.  SELL-64 with the window sorts its
     * rows inside windows of 1024 rows by default (sort_window), so that a
     * tile of 1024 sorted rows holds the rows of one row range; its slices
     * wider than 128 columns are read by the whole workgroup in chunks. */
    int32_t x_window;
    /* CSR: rows per lane group, 0 (choose by timing), 1, 2 or 4 */
    int32_t csr_rows;
    /* CSR: apply kernel, a spmv_csr_kernel.  The balanced kernel cuts the
     * entries into equal chunks of 512 per wave, sums the row segments of
     * each chunk with a segmented scan over the lanes and adds rows that
     * cross chunks with atomics after a pass that writes beta * y.  With
     * x_window it stages x in LDS like the HEC tail.  HEC: the kernel of
     * the tail -- balanced as above, or the vector kernel over the rows that
     * hold tail entries (each adds its sum onto the ELL part's result, no
     * atomics), or the column slices over the tail's rows; auto times the
     * vector and balanced ones, keeps the balanced one when the LDS window
     * is on, and times the column slices as the CSR format does.  HYB: the
     * balanced kernel over the COO tail, or the column slices (auto times
     * them as for HEC); the vector kernel is not a HYB tail kernel and is
     * ignored there. */
    int32_t csr_kernel;
    /* Windowed sorting: the pJDS sort of "Sparse matrix-vector multiplication
     * on GPGPU clusters" (Sect. 2.2: rows ordered by length, longest first)
     * applied only inside aligned windows of sort_window rows, so that rows
     * move less than a window and neighbouring rows keep reading
     * neighbouring x.
     *   SELL-64: -1 (default) sorts inside windows of 8192 rows (64 KiB of
     *            fp64 y: the y writes of a window stay within a few L2
     *            lines per slice and banded matrices keep their x
     *            locality), or of 1024 rows with the LDS window (x_window);
     *            0 keeps the row order; k >= 1 sorts inside windows of k
     *            rows, k >= n sorts all rows at once (the page's pJDS).
     *            Each slice is padded to its longest row.
     *   HYB/HEC: the rows of every 1024-row block of the ELL part;
     *            -1 (default) sorts inside the whole block when waves of 64
     *            unsorted rows would read more than 10% padding slots, 0 never,
     *            k in {64, 128, 256, 512, 1024} inside windows of k rows.
     *            The ELL part then keeps a position -> row permutation.
     *   ELL-R / CSR: must be -1 or 0. */
    int32_t sort_window;
    /* SELL-64: 1 stores the matrix of the permuted basis, P A P^T with
     * (P v)[r] = v[perm[r]] (perm = spmv_export SPMV_A_SELL_PERM): spmv_apply
     * then takes x and y in sorted row order (x'[r] = x[perm[r]]) and writes y
     * without the scatter through the permutation -- the form in which
     * "Sparse matrix-vector multiplication on GPGPU clusters" (Sect. 2.2) runs
     * a whole solve.  spmv_permute moves vectors between the bases.  0: the
     * caller's basis.  Must be 0 for the other formats. */
    int32_t permuted_basis;
    /* ELL-R / HYB / HEC without the LDS window: wave groups per tile of 64
     * rows ("Sparse Linear Algebra on AMD and NVIDIA GPUs -- The Race Is On":
     * the lanes of a group read one column of consecutive rows, several
     * groups share the rows).  0 chooses: 16 below 128 tiles of 64 rows
     * (rows of at least 256 entries), 4 below 512 tiles (rows of at least 16
     * entries), else 1; or 1, 4, 16. */
    int32_t ell_groups;
    /* Largest device footprint a padded format (ELL-R) may take, in bytes;
     * 0 means 75% of the device's memory. */
    uint64_t footprint_budget_bytes;
    /* CSR vector kernel: copy the entries of each wave's rows into LDS with
     * whole-line loads before the group sums (subwave 2..16, one row per
     * group).  The LDS slice of a wave holds the entries of 99.5 % of the
     * waves (at most 1,280 fp64 / 2,048 fp32 entries); the other waves read
     * directly.  The sums are the same either way.  -1 times both, 0 off,
     * 1 on. */
    int32_t csr_stage;
    /* Cache policy of the column indices (ELL-R, whose records hold value
     * and column together, SELL-64, the ELL part of HYB/HEC, the staged CSR
     * copy): 0 streams them past the caches like the values, 1 keeps them
     * (ELL-R: the records) in the caches (when they fit the last-level cache
     * beside x they stay there over applies that follow one another with
     * nothing else in between), -1 (default) streams them: with other work
     * between two applies (a solver's vector updates, other matrices) the
     * cached indices do not survive, and streaming is then the faster. */
    int32_t col_cache;
} spmv_convert_opts;

/* description of a handle (spmv_info) */
typedef struct {
    int64_t n;             /* rows = columns */
    int64_t nnz;           /* stored entries (duplicates and zeros kept) */
    int32_t dtype;         /* spmv_dtype */
    int32_t format;        /* active spmv_format */
    int32_t max_len;       /* longest row */
    int32_t ell_width;     /* ELL-R: max_len; HYB/HEC: K; otherwise 0 */
    int64_t tail_nnz;      /* HYB/HEC: entries outside the ELL part */
    int64_t ell_stride;    /* ELL-R / HYB / HEC: slots between consecutive
                              entries of a row (rows per column-major block):
                              ELL-R 64 * ceil(n / 64), HYB/HEC 1024 */
    int64_t slots;         /* stored slots of the active format incl. padding */
    int32_t subwave;       /* CSR: lanes per row */
    int32_t nslices;       /* SELL-64: slices */
    uint64_t footprint_bytes; /* device bytes held by the handle */
    int32_t x_window;      /* 1 when the active format stages x in LDS */
    int32_t csr_rows;      /* CSR: rows per lane group (1, 2 or 4) */
    int32_t csr_kernel;    /* CSR: SPMV_CSR_VECTOR or SPMV_CSR_BALANCED */
    int32_t permuted_basis; /* SELL-64: 1 when apply works in the sorted basis */
    int32_t ell_groups;    /* ELL-R / HYB / HEC: wave groups per 64-row tile */
    int32_t sort_window;   /* SELL-64 / HYB / HEC: rows per sort window in
                              effect (0: rows kept in order; SELL-64 with
                              all rows sorted at once reports n) */
    double band_fraction;  /* share of entries within the window's reach
                              (computed by ELL-R / SELL-64 / HYB / HEC
                              conversions) */
    int64_t ell_rows;      /* ELL-R / HYB / HEC: rows padded to whole blocks */
    int32_t csr_stage_slots; /* CSR vector kernel staged in LDS: entries one wave
                                can stage (0: the kernel reads directly) */
    int32_t tail_kernel;   /* HYB / HEC with tail entries: SPMV_CSR_BALANCED,
                              SPMV_CSR_XBLOCK or (HEC only) SPMV_CSR_VECTOR;
                              otherwise 0 */
    int32_t tail_subwave;  /* HEC vector tail: lanes per row, rows per lane */
    int32_t tail_rows;     /* group and LDS slots per wave (0: direct); */
    int32_t tail_stage_slots; /* all 0 otherwise */
    int32_t col_cached;    /* 1 when the active kernels keep col in the caches */
    int32_t ell_head;      /* ELL-R with the x window: slots of every row the
                              window kernel takes; the ell_long_rows longer rows
                              get the rest from a wave each (0: no split) */
    int64_t ell_long_rows;
} spmv_info_t;

/* arrays readable with spmv_export */
typedef enum {
    SPMV_A_ROWPTR = 0,     /* CSR row pointer, int32[n+1] */
    SPMV_A_COL = 1,        /* CSR columns, int32[nnz] */
    SPMV_A_VAL = 2,        /* CSR values, dtype[nnz] */
    SPMV_A_ELL_COL = 3,    /* ELL-R / ELL part: int32[width * ell_rows] in
                              column-major blocks of B = ell_stride rows: entry j
                              of row i at (i / B) * width * B + j * B + i % B
                              (ELL-R: a single block, B = 64 * ceil(n / 64);
                              HYB/HEC: B = 1024).  ELL-R stores each slot as a
                              (value, column) record; its columns and values
                              are exported as these two arrays */
    SPMV_A_ELL_VAL = 4,    /* dtype[width * ell_rows]; pad slots col 0, value +0 */
    SPMV_A_ELL_LEN = 5,    /* int32[ell_rows]: entries of each row held in ELL */
    SPMV_A_SELL_PERM = 6,  /* int32[n]: original row at sorted position r */
    SPMV_A_SELL_SLICE_PTR = 7, /* int64[nslices+1]: first slot of each slice */
    SPMV_A_SELL_LEN = 8,   /* int32[64 * nslices]: length of sorted row r */
    SPMV_A_SELL_COL = 9,   /* int32[slots]: entry j of sorted row r at
                              slice_ptr[r/64] + 64*j + r%64 */
    SPMV_A_SELL_VAL = 10,  /* dtype[slots] */
    SPMV_A_TAIL_ROW = 11,  /* HYB: int32[tail_nnz] row of each tail entry */
    SPMV_A_TAIL_PTR = 12,  /* HEC: int32[n+1] start of each row's tail */
    SPMV_A_TAIL_COL = 13,  /* HYB/HEC: int32[tail_nnz] */
    SPMV_A_TAIL_VAL = 14,  /* HYB/HEC: dtype[tail_nnz] */
    SPMV_A_ELL_PERM = 15   /* HYB/HEC with a sorted ELL part: int32[ell_rows],
                              row at each position (itself for padding) */
} spmv_array;

/*
 * spmv_create -- copy a matrix onto the device and validate it.
 *
 *   out        host out-parameter: the new handle (set only on success)
 *   kind       SPMV_IN_CSR: `rowidx` is the CSR row pointer, int64[n+1];
 *              SPMV_IN_COO: `rowidx` is the row of every entry, int64[nnz]
 *              (any order; entries are ordered by (row, input position),
 *              which keeps the input order inside a row)
 *   n, nnz     matrix size and stored entries (0 <= n < 2^31 - 1,
 *              0 <= nnz <= 2^31 - 65537)
 *   rowidx     device pointer as above (may be NULL only if COO and nnz == 0)
 *   col        device int32[nnz], may be NULL when nnz == 0
 *   val        device dtype[nnz], may be NULL when nnz == 0
 *   dtype      SPMV_F32 or SPMV_F64
 *   stream     the work is ordered on this stream; the call synchronises it
 *              before returning, after which the caller may free its arrays
 *
 * Duplicated (row, col) pairs and explicit zeros are kept and summed by
 * apply; columns need not be sorted.  The handle owns device copies (CSR with
 * int32 row pointer).  The active format is SPMV_CSR.
 * Errors: INVALID_ARG, INVALID_MATRIX (nothing allocated is kept), NO_MEMORY,
 * HIP.
 */
int spmv_create(spmv_t *out, int kind, int64_t n, int64_t nnz,
                const int64_t *rowidx, const int32_t *col, const void *val,
                int dtype, void *stream);

/*
 * spmv_convert -- build `format` on the device from the CSR copy and make it
 * the active format.  Synchronous (small size read-backs are needed).
 * The previous non-CSR format is released once the new one is built; on any
 * error the handle is left exactly as it was.  Converting to SPMV_CSR
 * switches the active format and chooses its kernel (see csr_kernel).
 * SPMV_AUTO releases the previous format before it starts and leaves CSR
 * active if it fails.
 *   opts  may be NULL (defaults, see spmv_convert_opts)
 * Errors: STATE, INVALID_ARG (unknown format, bad subwave), FOOTPRINT (the
 * padded layout exceeds the budget; e.g. ELL-R of a matrix with a few very
 * long rows), NO_MEMORY, HIP.
 */
int spmv_convert(spmv_t h, int format, const spmv_convert_opts *opts);

/*
 * spmv_apply -- y = alpha * A * x + beta * y with the active format.
 *   y      device dtype[n], read only when beta != 0, always written
 *   x      device dtype[n]; must not overlap y
 *   alpha, beta  scalars (rounded to float for SPMV_F32 handles)
 *   stream the kernels are enqueued on this stream; no host synchronisation
 * Accumulation is in the handle's dtype with fused multiply-adds; HYB/HEC,
 * split SELL slices and the balanced CSR kernel add partial sums with
 * atomics in global memory, and the column-slice CSR kernel adds them with
 * atomics in LDS, so their last bits may vary between runs.  Errors: STATE, INVALID_ARG (null or overlapping
 * vectors), HIP (launch failure).
 */
int spmv_apply(spmv_t h, void *y, const void *x, double alpha, double beta,
               void *stream);

/*
 * spmv_permute -- move a vector between the caller's basis and the sorted
 * basis of the active SELL-64 format (the permutation of its rows, with or
 * without permuted_basis):
 *   direction 0: dst[r] = src[perm[r]]   (caller's basis -> sorted)
 *   direction 1: dst[perm[r]] = src[r]   (sorted -> caller's basis)
 *   dst, src  device dtype[n], must not overlap
 * Asynchronous on `stream`; moves the values exactly.
 * Errors: STATE (null handle, active format not SELL-64), INVALID_ARG
 * (null pointer, overlap, bad direction), HIP.
 */
int spmv_permute(spmv_t h, void *dst, const void *src, int direction, void *stream);

/* Krylov solvers over spmv_apply ("Development of Krylov and AMG linear
 * solvers for large-scale sparse matrices on GPUs", Sect. 3: the solvers the
 * sparse product serves) */
typedef enum {
    SPMV_SOLVE_CG = 0,       /* conjugate gradients: A symmetric positive definite */
    SPMV_SOLVE_BICGSTAB = 1  /* BiCGSTAB (van der Vorst): general A */
} spmv_solve_method;

typedef struct {
    int32_t method;     /* spmv_solve_method */
    int32_t max_iter;   /* iteration cap (> 0) */
    double rtol;        /* stop when ||r|| <= rtol * ||b|| (2-norms, recurred
                           residual r) */
} spmv_solve_opts;

typedef struct {
    int32_t iterations;   /* iterations taken */
    int32_t converged;    /* 1 when ||r|| <= rtol * ||b|| */
    double rel_residual;  /* ||r|| / ||b|| (||r|| when b = 0) */
} spmv_solve_info;

/*
 * spmv_solve -- solve A x = b with the active format's apply.
 *   x     device dtype[n]: the initial guess on entry, the solution on return
 *   b     device dtype[n], must not overlap x
 *   opts  method, iteration cap, relative tolerance
 *   info  host out-parameter (may be NULL)
 * Vector updates are fused kernels; inner products are fp64 sums in a fixed
 * order.  The iteration's scalars stay on the device and batches of eight
 * iterations are replayed from a HIP graph on a private stream (ordered
 * after `stream`'s earlier work); the call returns when the solve is done.
 * Work vectors (3 n for CG, 6 n for BiCGSTAB) are allocated for the call.
 * Not reaching the tolerance is not an error (info->converged = 0).
 * Errors: STATE, INVALID_ARG (null pointer, overlap, bad method / cap /
 * tolerance), NO_MEMORY, HIP.
 */
int spmv_solve(spmv_t h, void *x, const void *b, const spmv_solve_opts *opts,
               spmv_solve_info *info, void *stream);

/*
 * spmv_solve_noalloc -- spmv_solve for callers that cannot allocate device
 * memory (serving loops that must not call hipMalloc, harnesses that forbid
 * allocation): the same method, options, iterates and results, with no
 * device allocation and no stream or graph created.
 *   x, b, opts, info, stream  as for spmv_solve; the handle's device must be
 *                             the current device
 * The work vectors, inner-product partial sums and iteration scalars live in
 * one array of 64 MiB that the library keeps per GPU until the process ends
 * (taken at the first call on each device).  The vectors must fit it:
 * 3 (CG) or 6 (BiCGSTAB) vectors of n entries, each rounded up to 256 bytes,
 * in 64 MiB - 64 KiB -- e.g. fp64 CG up to 2,793,472 rows, fp64 BiCGSTAB up
 * to 1,396,736, fp32 twice as many; larger n gives INVALID_ARG.  Batches of
 * eight iterations are enqueued on `stream` itself and the host reads the
 * done flag after each batch; the call returns when the solve is done.
 * Every call on one GPU uses that GPU's one array, and each call sets up all
 * of it that it reads: calls that overlap in time on one GPU (other threads)
 * race and must not be made.
 * Errors: as spmv_solve (never NO_MEMORY from an allocation of its own), plus
 * INVALID_ARG when n exceeds the limit above and STATE when the handle's
 * device is not current.
 */
int spmv_solve_noalloc(spmv_t h, void *x, const void *b, const spmv_solve_opts *opts,
                       spmv_solve_info *info, void *stream);

/* spmv_destroy -- free every device buffer of the handle (synchronises the
 * device first).  A NULL handle is accepted.  The handle is released even
 * when HIP is returned (an earlier asynchronous error reported by the
 * synchronisation); it must not be used again.  Errors: HIP. */
int spmv_destroy(spmv_t h);

/*
 * spmv_info -- fill *out (host) with the handle's description.
 * Errors: STATE, INVALID_ARG.
 */
int spmv_info(spmv_t h, spmv_info_t *out);

/*
 * spmv_export -- copy one of the handle's device arrays to host memory
 * (synchronous).  With host_dst == NULL only *bytes is set.  The array must
 * belong to the active format (or to CSR).  capacity_bytes below the
 * array's size gives INVALID_ARG.  Errors: STATE (array not present),
 * INVALID_ARG, HIP.
 */
int spmv_export(spmv_t h, int array, void *host_dst, int64_t capacity_bytes,
                int64_t *bytes);

/*
 * spmv_stream_copy -- dst[0..bytes) = src[0..bytes) with 16-byte
 * nontemporal loads and stores, one per thread over a grid that covers the
 * buffer (the fastest copy shape measured on MI355X); the reference
 * bandwidth that the SpMV kernels are compared with.  dst == NULL reads
 * src only (the whole 16-byte words of it) and writes nothing: the
 * bandwidth of loads alone, for read-dominated kernels.  Both device
 * pointers must be 16-byte aligned and not overlap.  Asynchronous on stream.
 * Errors: INVALID_ARG, HIP.
 */
int spmv_stream_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* spmv_last_error -- message of the calling thread's last failed call
 * ("" if none).  The pointer stays valid until that thread's next call. */
const char *spmv_last_error(void);

/* spmv_version -- library version string */
const char *spmv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPMV_AMD_H */
