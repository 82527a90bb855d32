// Host tests of the kernels' index arithmetic (sparse_formats_amd/csrc/
// index_math.h), run under AddressSanitizer and UndefinedBehaviorSanitizer
// (signed overflow aborts): the same functions the kernels call, at the
// boundaries of the 32-bit and 64-bit ranges where the largest matrices put
// them (rows and entries near 2^31, ELL slot offsets past 2^32, grids at the
// dispatch limit), and exhaustively or against plain definitions on small
// cases.  Prints "index_math: all N checks passed" and exits 0, or names the
// first failed check and exits 1.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../sparse_formats_amd/csrc/index_math.h"

using namespace spmv;

static long g_checks = 0;

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        ++g_checks;                                                        \
        if (!(cond)) {                                                     \
            std::fprintf(stderr, "FAILED %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                             \
            std::fprintf(stderr, "\n");                                    \
            std::exit(1);                                                  \
        }                                                                  \
    } while (0)

// row pointers of a matrix whose rows r >= first have `len` entries each,
// computed on demand (the largest matrices do not fit the host)
struct VirtualPtr {
    int64_t first, base, len;
    int64_t operator[](int64_t r) const { return base + (r - first) * len; }
};

static void test_xcd_tile() {
    // a bijection of [0, grid) that gives XCD k the k-th contiguous eighth
    for (int64_t grid = 1; grid <= 300; ++grid) {
        std::vector<int> seen(grid, 0);
        for (int64_t b = 0; b < grid; ++b) {
            const int64_t t = xcd_tile(b, grid);
            CHECK(t >= 0 && t < grid, "grid %lld b %lld -> %lld", (long long)grid, (long long)b,
                  (long long)t);
            seen[t]++;
            if (b >= 8) CHECK(t == xcd_tile(b - 8, grid) + 1, "contiguous per XCD");
        }
        for (int64_t t = 0; t < grid; ++t) CHECK(seen[t] == 1, "grid %lld tile %lld", (long long)grid, (long long)t);
    }
    // the largest grids launched: 2^31 - 1 workgroups (dispatch limit)
    for (int64_t grid : {int64_t(INT_MAX), int64_t(INT_MAX) - 5, int64_t(1) << 26}) {
        for (int64_t b : {int64_t(0), int64_t(7), int64_t(8), grid / 2, grid - 9, grid - 8, grid - 1}) {
            const int64_t t = xcd_tile(b, grid);
            CHECK(t >= 0 && t < grid, "large grid %lld b %lld", (long long)grid, (long long)b);
        }
        // the first tile of each XCD follows the last tile of the previous one
        for (int64_t k = 0; k < 7; ++k) {
            int64_t last = -1;  // last dispatch of XCD k
            for (int64_t b = grid - 1; b >= 0 && last < 0; --b)
                if ((b & 7) == k) last = b;
            CHECK(xcd_tile(last, grid) + 1 == xcd_tile(k + 1, grid), "XCD %lld boundary", (long long)k);
        }
    }
}

static void test_ell_row_base() {
    // ELL-R: one block of pad64(n) rows; HYB/HEC: blocks of 1024 rows
    const int64_t n = int64_t(INT_MAX) - 2, S = (n + 63) / 64 * 64;
    for (int64_t i : {int64_t(0), int64_t(1), n / 2, n - 1, S - 1}) {
        CHECK(ell_row_base(i, S, 2000 * S) == i, "ELL-R row %lld", (long long)i);
        for (int64_t W : {int64_t(1), int64_t(40), int64_t(2000), int64_t(50000)}) {
            const __int128 ref = (__int128)(i / 1024) * W * 1024 + i % 1024;
            CHECK((__int128)ell_row_base(i, 1024, W * 1024) == ref, "blocked row %lld W %lld",
                  (long long)i, (long long)W);
            // the last slot of the row stays below the array's end
            const __int128 last = ref + (__int128)(W - 1) * 1024;
            const __int128 end = (__int128)((n + 1023) / 1024) * 1024 * W;
            CHECK(last < end && last < ((__int128)1 << 62), "slot range");
        }
    }
}

static void test_row_of() {
    // small: every entry of random pointer arrays with empty rows
    std::mt19937_64 rng(7);
    for (int trial = 0; trial < 300; ++trial) {
        const int n = 1 + rng() % 60;
        std::vector<int> ptr(n + 1, 0);
        for (int r = 0; r < n; ++r) ptr[r + 1] = ptr[r] + (rng() % 3 == 0 ? 0 : rng() % 5);
        for (int e = 0; e < ptr[n]; ++e) {
            int ref = 0;
            while (ptr[ref + 1] <= e) ++ref;
            const int got = row_of(ptr.data(), 0, n - 1, e);
            CHECK(got == ref, "trial %d entry %d: %d vs %d", trial, e, got, ref);
        }
    }
    // the last rows of a matrix with 2^31 - 2 rows: lo + hi would pass 2^31
    const int64_t n = int64_t(INT_MAX) - 2;
    const VirtualPtr vp{0, 0, 1};  // one entry per row: row r holds entry r
    for (int64_t e : {n - 1, n - 2, n - 1000, int64_t(1) << 30}) {
        const int got = row_of(vp, (int)(n - 4096 > e ? e - 10 : n - 4096), (int)(n - 1), e);
        CHECK(got == e, "row of entry %lld: %d", (long long)e, got);
    }
    // rows of 21 entries up to nnz = 2^31 - 65537 (the library's cap)
    const int64_t nnz = (int64_t(1) << 31) - 65537, rows = nnz / 21;
    const VirtualPtr v21{0, 0, 21};
    for (int64_t e : {nnz - 1 - nnz % 21, rows * 21 - 1, int64_t(21) * (rows / 2)}) {
        const int got = row_of(v21, 0, (int)(rows - 1), e);
        CHECK(got == e / 21, "entry %lld", (long long)e);
    }
}

static void test_run_next_start() {
    // a lane run starting in row cur, the next run in row hi: the next row
    // starts read are clamped to hi + 1, so no index passes n
    const int n = INT_MAX - 2;  // rows 0 .. n - 1, ptr[n] exists
    for (int cur : {0, 5, n - 9, n - 2, n - 1})
        for (int64_t hi64 : {int64_t(cur), int64_t(cur) + 1, int64_t(cur) + 3, int64_t(cur) + 100})
            for (int j = 0; j < 8; ++j) {
                if (hi64 > n - 1) continue;
                const int hi = (int)hi64;
                const int idx = run_next_start(cur, hi, j);
                CHECK(idx <= hi + 1 && idx >= cur + 1 && idx <= n, "cur %d hi %d j %d -> %d", cur, hi,
                      j, idx);
                if (j < hi - cur) CHECK(idx == cur + 1 + j, "unclamped");
            }
}

static void test_xblk_ranges() {
    // candidate starts: the row holding entry r * nnz / R0, against a linear
    // search, on random row pointers (empty rows too) and at n near 2^31
    std::mt19937_64 rng(11);
    for (int trial = 0; trial < 2000; ++trial) {
        const int n = 1 + (int)(rng() % 300);
        std::vector<int> ptr(n + 1, 0);
        for (int i = 0; i < n; ++i) ptr[i + 1] = ptr[i] + (rng() % 3 == 0 ? 0 : (int)(rng() % 9));
        const int64_t nnz = ptr[n], R0 = 1 + (int64_t)(rng() % 40);
        std::vector<int> cand(R0 + 1);
        for (int64_t r = 0; r <= R0; ++r) {
            cand[r] = xblk_bound(ptr.data(), n, nnz, r, R0);
            if (r == 0) CHECK(cand[r] == 0, "first start");
            else if (r == R0) CHECK(cand[r] == n, "last start");
            else if (nnz > 0) {
                const int64_t e = r * nnz / R0;
                int ref = 0;
                for (int i = 0; i < n; ++i)
                    if (ptr[i] <= e) ref = i;
                CHECK(cand[r] == ref, "trial %d r %lld: %d vs %d", trial, (long long)r, cand[r], ref);
            }
            if (r > 0) CHECK(cand[r] >= cand[r - 1], "candidates non-decreasing");
        }
        // ranges: strictly increasing starts from 0 to n, at most cap rows,
        // every distinct candidate kept as a start
        const int cap = 1 + (int)(rng() % 50);
        const int64_t R = xblk_split_ranges(cand.data(), R0, cap, nullptr);
        std::vector<int> out(R + 1, -1);
        CHECK(xblk_split_ranges(cand.data(), R0, cap, out.data()) == R, "count twice");
        CHECK(out[0] == 0 && out[R] == n, "ranges cover [0, n)");
        for (int64_t k = 0; k < R; ++k)
            CHECK(out[k] < out[k + 1] && out[k + 1] - out[k] <= cap, "range %lld", (long long)k);
        for (int64_t r = 0; r < R0; ++r) {
            bool found = false;
            for (int64_t k = 0; k <= R; ++k) found |= out[k] == cand[r];
            CHECK(found, "candidate %lld kept", (long long)r);
        }
    }
    // n near 2^31 (the column-slice kernel takes fewer rows, the helpers not):
    // every row one entry but the first, which holds nnz - (n - 1)
    {
        const int n = INT_MAX - 1;
        const int64_t nnz = (int64_t)INT_MAX - 65536;
        struct P {
            int n;
            int64_t nnz;
            int64_t operator[](int64_t i) const { return i == 0 ? 0 : nnz - (n - i); }
        } ptr{n, nnz};
        const int64_t R0 = 256 * 410;
        int prev = 0;
        for (int64_t r = 0; r <= R0; r += 997) {
            const int c = xblk_bound(ptr, n, nnz, r, R0);
            CHECK(c >= prev && c <= n, "r %lld -> %d", (long long)r, c);
            if (r > 0 && r < R0) {
                const int64_t e = r * nnz / R0;
                CHECK(ptr[c] <= e && e < ptr[c + 1], "row of entry %lld", (long long)e);
            }
            prev = c;
        }
        // one stretch of n rows in pieces of at most 20480
        const int cand[2] = {0, n};
        const int64_t R = xblk_split_ranges(cand, 1, 20480, nullptr);
        CHECK(R == ((int64_t)n + 20479) / 20480, "pieces %lld", (long long)R);
        std::vector<int> out(R + 1);
        xblk_split_ranges(cand, 1, 20480, out.data());
        for (int64_t k = 0; k < R; ++k)
            CHECK(out[k] < out[k + 1] && out[k + 1] - out[k] <= 20480, "piece %lld", (long long)k);
    }
    // count positions: a bijection of [0, kS n) onto the counts of (row, slice),
    // slice-major inside each range, tiles starting at xblk_slot(rb, nr, b, rb)
    for (int trial = 0; trial < 200; ++trial) {
        const int n = 1 + (int)(rng() % 500), kS = 8;
        std::vector<int> starts = {0};
        while (starts.back() < n) starts.push_back(std::min(n, starts.back() + 1 + (int)(rng() % 60)));
        std::vector<char> seen((size_t)kS * n, 0);
        for (size_t r = 0; r + 1 < starts.size(); ++r) {
            const int rb = starts[r], nr = starts[r + 1] - rb;
            for (int b = 0; b < kS; ++b)
                for (int i = rb; i < rb + nr; ++i) {
                    const int64_t s = xblk_slot(rb, nr, b, i, kS);
                    CHECK(s >= 0 && s < (int64_t)kS * n && !seen[s], "slot of row %d slice %d", i, b);
                    seen[s] = 1;
                    CHECK(s == xblk_slot(rb, nr, b, rb, kS) + (i - rb), "tile order");
                    if (i == rb && b > 0)
                        CHECK(s == xblk_slot(rb, nr, b - 1, rb + nr - 1, kS) + 1, "tiles adjacent");
                }
        }
    }
    // the largest slot: kS n - 1 < 2^31 for n up to (2^31 - 17) / 8
    {
        const int64_t n = ((int64_t)INT_MAX - 16) / 8, rb = n - 20480, nr = 20480;
        CHECK(xblk_slot(rb, nr, 7, n - 1, 8) == 8 * n - 1, "last slot");
        CHECK(8 * n - 1 <= (int64_t)INT_MAX, "fits int");
    }
}

static void test_xblk_tiles() {
    // tile of an entry against the plain definition: band tile kS when the
    // column lies within band of the range's rows, else its slice; no band
    // tile when band < 0
    std::mt19937_64 rng(13);
    for (int trial = 0; trial < 200000; ++trial) {
        const int64_t n = 1 + (int64_t)(rng() % (trial & 1 ? (1u << 28) : 5000));
        const int64_t width = (n + 7) / 8, nr = 1 + (int64_t)(rng() % std::min<int64_t>(n, 20480));
        const int64_t rb = (int64_t)(rng() % (uint64_t)(n - nr + 1));
        const int64_t band = trial % 3 == 0 ? -1 : (int64_t)(rng() % 60000);
        const int64_t c = (int64_t)(rng() % (uint64_t)n);
        const int t = xblk_tile(c, rb, nr, band, width, 8);
        const bool near = band >= 0 && c >= rb - band && c < rb + nr + band;
        CHECK(t == (near ? 8 : (int)(c / width)), "tile of column %lld", (long long)c);
        CHECK(t >= 0 && t <= 8, "tile in range");
    }
    // packing: every column of the band of a range of at most cap rows and
    // every row offset below cap survive the 32-bit word, at both dtypes'
    // widths, with the band's first column below 0 and the last near 2^28
    const int lbs[2] = {15, 16};
    const int64_t caps[2] = {20480, 40960};
    for (int k = 0; k < 2; ++k) {
        const int lb = lbs[k];
        const int64_t cap = caps[k], band = xblk_band(lb, cap);
        CHECK(band > 0 && cap + 2 * band <= ((int64_t)1 << (32 - lb)), "band %lld", (long long)band);
        CHECK(cap <= ((int64_t)1 << lb), "row offsets fit");
        const int64_t n = ((int64_t)INT_MAX - 16) / 9;
        const int64_t rbs[3] = {0, 777, n - cap};
        for (int64_t rb : rbs) {
            const int64_t lo = rb - band, hi = rb + cap + band;  // columns [lo, hi)
            for (int64_t c : {lo, lo + 1, rb, rb + cap / 2, hi - 2, hi - 1})
                for (int lr : {0, 1, (int)cap / 3, (int)cap - 1}) {
                    const uint32_t w = xblk_pack(c, rb, band, lr, lb);
                    CHECK(xblk_unpack_col(w, rb, band, lb) == c, "column %lld", (long long)c);
                    CHECK((int)(w & ((1u << lb) - 1)) == lr, "row offset %d", lr);
                    // the kernel's form: 32-bit band start plus the shifted word
                    if (rb - band >= INT_MIN && c < INT_MAX)
                        CHECK((int64_t)((int)(rb - band) + (int)(w >> lb)) == c, "int form");
                }
        }
    }
}

static void test_in_window() {
    // the window conversions take n < 2^31 - 1 - 2 WL (WL = 40,960 fp32 entries)
    const int WL32 = 40960, WL64 = 20480;
    const int nmax = INT_MAX - 2 * WL32 - 1;
    for (int WL : {WL32, WL64}) {
        const int lead = (WL - 1024) / 2;
        for (int wl : {-lead, 0, nmax - 1024 - lead, nmax})
            for (int q : {0, 1, nmax - 1, wl + WL - 1, wl + WL, wl < 0 ? 0 : wl}) {
                if (q < 0 || q >= nmax) continue;
                const bool ref = (int64_t)q >= wl && (int64_t)q < (int64_t)wl + WL;
                CHECK(in_window(q, wl, WL) == ref, "q %d wl %d WL %d", q, wl, WL);
            }
    }
}

static void test_sell_chunks() {
    std::mt19937_64 rng(13);
    for (int trial = 0; trial < 2000; ++trial) {
        const int ns = 1 + (int)(rng() % 6);
        std::vector<int> len(64 * ns);
        std::vector<int64_t> sp(ns + 1, 0);
        for (int q = 0; q < ns; ++q) {
            int w = 0;
            for (int l = 0; l < 64; ++l) {
                const int x = rng() % 5 == 0 ? (int)(rng() % 700) : (int)(rng() % 40);
                len[64 * q + l] = x;
                w = x > w ? x : w;
            }
            sp[q + 1] = sp[q] + 64 * (int64_t)w;
        }
        for (int groups = 0; groups < 2; ++groups) {
            const int split = groups ? 128 : 256, head = groups ? 64 : 0, chunk = 128;
            for (int q = 0; q < ns; ++q) {
                const int c = sell_slice_chunks(q, sp.data(), len.data(), split, head, chunk,
                                                groups, nullptr);
                std::vector<int4> out(c + 1);
                CHECK(sell_slice_chunks(q, sp.data(), len.data(), split, head, chunk, groups,
                                        out.data()) == c, "count twice");
                // every (row, column) past `head` of a wide slice is in exactly one
                // chunk that covers its row
                const int w = (int)((sp[q + 1] - sp[q]) / 64);
                for (int l = 0; l < 64; ++l)
                    for (int j = 0; j < len[64 * q + l]; ++j) {
                        int hits = 0;
                        for (int k = 0; k < c; ++k) {
                            const int4 ch = out[k];
                            const bool row_in = !groups || l / 16 == ch.w;
                            hits += ch.x == q && row_in && j >= ch.y && j < ch.z;
                        }
                        const bool want = w > split && j >= head;
                        CHECK(hits == (want ? 1 : 0), "trial %d q %d row %d col %d hits %d", trial, q,
                              l, j, hits);
                    }
                for (int k = 0; k < c; ++k) CHECK(out[k].z - out[k].y <= chunk && out[k].z <= w, "chunk range");
            }
        }
    }
}

static void test_launch_pieces() {
    // a dispatch covers fewer than 2^32 work-items and 2^31 - 1 workgroups
    const int64_t max_items = int64_t(1) << 31;
    for (int threads : {64, 256, 64 * 4, 64 * 16, 1024}) {
        const int64_t per = blocks_per_piece(max_items, threads);
        CHECK(per * threads <= max_items && (per + 1) * threads > max_items, "threads %d", threads);
        CHECK(per <= INT_MAX, "grid limit");
        // the pieces of the largest launch (2^31 - 2 rows, a lane group per row)
        const int64_t blocks = (int64_t(INT_MAX) - 2) * 64 / threads + 1;
        int64_t covered = 0;
        for (int64_t b0 = 0; b0 < blocks; b0 += per) {
            const int64_t nb = blocks - b0 < per ? blocks - b0 : per;
            CHECK(nb * threads < (int64_t(1) << 32), "piece size");
            CHECK(b0 + xcd_tile(nb - 1, nb) < blocks && b0 + xcd_tile(0, nb) >= b0, "piece tiles");
            covered += nb;
        }
        CHECK(covered == blocks, "pieces cover the grid");
    }
}

int main() {
    test_xcd_tile();
    test_ell_row_base();
    test_row_of();
    test_run_next_start();
    test_xblk_ranges();
    test_xblk_tiles();
    test_in_window();
    test_sell_chunks();
    test_launch_pieces();
    std::printf("index_math: all %ld checks passed\n", g_checks);
    return 0;
}
