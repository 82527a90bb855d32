// Device helpers shared by the gfx950 SpMV kernels: XCD-aware block order,
// streaming loads, cross-lane sums on wave64 and fp atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "index_math.h"

namespace spmv {

constexpr int kWave = 64;
// A dispatch covers fewer than 2^32 work-items; launches of kernels whose
// grids grow with the row count are split into pieces of at most this many
// work-items (each piece passes its first tile).
constexpr int64_t kMaxLaunchItems = int64_t(1) << 31;
// cache-policy bits of a memory instruction on gfx950: nontemporal
constexpr int kCachePolicyNT = 2;

// Streaming (non-temporal) loads for matrix data that is read exactly once
// per apply, so it does not evict x from the caches.
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
    return __builtin_nontemporal_load(p);
}

// ELL slot records (ELLPACK-R and the ELL part of HYB/HEC): a slot's value and
// column side by side, 12 bytes in fp64 (4-byte aligned) and 8 in fp32, so a
// slot read on its own -- a long row's entries lie a whole column height
// apart -- costs one cache line instead of one for the value and one for the
// column.  kNT streams the record past the caches.
template <typename T>
constexpr int kRecInts = (int)sizeof(T) / 4 + 1;
typedef double rec_double __attribute__((aligned(4)));  // a record's value: 4-byte aligned
typedef float rec_float __attribute__((aligned(4)));
template <typename T>
struct RecVal;
template <>
struct RecVal<double> {
    typedef rec_double type;
};
template <>
struct RecVal<float> {
    typedef rec_float type;
};
template <typename T, bool kNT>
__device__ __forceinline__ void ld_rec(const int* rec, int64_t slot, T& v, int& c) {
    const int* p = rec + kRecInts<T> * slot;
    const typename RecVal<T>::type* pv = reinterpret_cast<const typename RecVal<T>::type*>(p);
    if constexpr (kNT) {
        v = __builtin_nontemporal_load(pv);
        c = __builtin_nontemporal_load(p + kRecInts<T> - 1);
    } else {
        v = *pv;
        c = p[kRecInts<T> - 1];
    }
}
// The record at byte offset `off` from a wave-uniform address: one scalar
// base and a 32-bit offset per lane (no 64-bit address per lane).
template <typename T, bool kNT>
__device__ __forceinline__ void ld_rec_at(const int* base, uint32_t off, T& v, int& c) {
    const char* b = reinterpret_cast<const char*>(base) + off;
    const typename RecVal<T>::type* pv = reinterpret_cast<const typename RecVal<T>::type*>(b);
    const int* pc = reinterpret_cast<const int*>(b + sizeof(T));
    if constexpr (kNT) {
        v = __builtin_nontemporal_load(pv);
        c = __builtin_nontemporal_load(pc);
    } else {
        v = *pv;
        c = *pc;
    }
}
template <typename T>
__device__ __forceinline__ void st_rec(int* rec, int64_t slot, T v, int c) {
    int* p = rec + kRecInts<T> * slot;
    *reinterpret_cast<typename RecVal<T>::type*>(p) = v;
    p[kRecInts<T> - 1] = c;
}

// Column indices: streamed like the values (kNT), or kept in the caches --
// when the index array fits the last-level cache beside x, it stays there
// over repeated applies (the format times both and keeps the faster).
template <bool kNT>
__device__ __forceinline__ int ld_col(const int* p) {
    if constexpr (kNT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// ---------------------------------------------------------------------------
// cross-lane moves.  DPP controls (gfx9 encoding):
//   quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2)
//   row_half_mirror = 0x141 (lane i <-> 7-i inside 8), row_mirror = 0x140
//   (lane i <-> 15-i inside 16).  After the sums of the smaller groups are
//   in every lane, a mirror pairs each lane with one of the other half, so
//   the butterfly stays a full reduction.
// ds_swizzle bit mode 0x401F: and_mask 0x1F, xor_mask 0x10 -> lane ^ 16
// inside each 32-lane half.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
    const int64_t b = __double_as_longlong(v);
    const int lo = dpp_i32<CTRL>((int)(b & 0xffffffff));
    const int hi = dpp_i32<CTRL>((int)(b >> 32));
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float swz16_move(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

__device__ __forceinline__ double swz16_move(double v) {
    const int64_t b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_ds_swizzle((int)(b & 0xffffffff), 0x401F);
    const int hi = __builtin_amdgcn_ds_swizzle((int)(b >> 32), 0x401F);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float lane_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ double lane_read(double v, int lane) {
    const int64_t b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffff), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Sum over aligned groups of S lanes (S a power of two, 1..64).  For S <= 32
// every lane of the group ends with the group sum; for S == 64 lane 0 holds
// the wave's sum.  All lanes of a group must be active.
template <int S, typename T>
__device__ __forceinline__ T group_sum(T v) {
    if constexpr (S >= 2) v += dpp_move<0xB1>(v);
    if constexpr (S >= 4) v += dpp_move<0x4E>(v);
    if constexpr (S >= 8) v += dpp_move<0x141>(v);
    if constexpr (S >= 16) v += dpp_move<0x140>(v);
    if constexpr (S >= 32) v += swz16_move(v);
    if constexpr (S >= 64) v += lane_read(v, 32);
    return v;
}

// DPP moves with an explicit value for lanes that have no source: lanes
// whose source lies outside the pattern (or whose row is not in ROWS) get
// `old`.  Controls (gfx9): row_shr:d = 0x110 + d inside rows of 16 lanes,
// row_bcast:15 = 0x142 (lane 15 of each row to the next row), row_bcast:31 =
// 0x143 (lane 31 to rows 2 and 3), wave_shr:1 = 0x138 (lane i - 1 across the
// wave), wave_shl:1 = 0x130 (lane i + 1).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or(float old, float v) {
    return __int_as_float(dpp_or<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_or(double old, double v) {
    const int64_t o = __double_as_longlong(old), b = __double_as_longlong(v);
    const int lo = dpp_or<CTRL, ROWS>((int)(o & 0xffffffff), (int)(b & 0xffffffff));
    const int hi = dpp_or<CTRL, ROWS>((int)(o >> 32), (int)(b >> 32));
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Segmented inclusive scan over the wave: lanes with equal keys form the
// segments (keys must be non-decreasing over the lanes and >= 0); each lane
// gets the sum of v over its segment up to itself.  Hillis-Steele steps of
// 1, 2, 4, 8 lanes inside rows of 16, then the last lane of row 0 (and 2)
// into rows 1 (and 3), then lane 31 into rows 2 and 3.  With monotone keys a
// source lane with the same key means every lane in between has it too, so
// each conditional add joins two adjacent pieces of one segment.
template <typename T>
__device__ __forceinline__ T segmented_scan(int key, T v) {
#define SPMV_SEG_STEP(CTRL, ROWS)                         \
    {                                                     \
        const int k2 = dpp_or<CTRL, ROWS>(-1, key);       \
        const T s2 = dpp_or<CTRL, ROWS>(T(0), v);         \
        if (k2 == key) v += s2;                           \
    }
    SPMV_SEG_STEP(0x111, 0xF)
    SPMV_SEG_STEP(0x112, 0xF)
    SPMV_SEG_STEP(0x114, 0xF)
    SPMV_SEG_STEP(0x118, 0xF)
    SPMV_SEG_STEP(0x142, 0xA)
    SPMV_SEG_STEP(0x143, 0xC)
#undef SPMV_SEG_STEP
    return v;
}

// Workgroup barrier for LDS hand-offs that leaves global loads in flight:
// waits only for this wave's LDS operations, then s_barrier.  A plain
// __syncthreads() also waits for every outstanding global load, which would
// drain the prefetch of the next step that the window kernels rely on.
// Orders a wave's LDS stores before its later LDS loads from other lanes of
// the same wave (data staged in a slice only that wave touches).  LDS
// operations of one wave complete in issue order, so no wait is needed; the
// fences keep the compiler from moving the loads above the stores.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16 bytes per lane straight from global memory into LDS (no registers):
// lane i's bytes land at lds + 16 * i, with `lds` the same for the whole wave.
// The copy is counted by vmcnt; wait_vm() waits for it.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// the same, without keeping the lines in the caches (data read once)
__device__ __forceinline__ void load_lds16_nt(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0,
                                     kCachePolicyNT);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Fill win with x[from, to) (element q at slot q mod WL): the loads of a
// thread are all issued before its stores, so the fill costs one latency.
template <typename T, int WL>
__device__ __forceinline__ void window_fill(T* win, const T* __restrict__ x, int64_t from,
                                            int64_t to) {
    constexpr int kPer = (WL + 1023) / 1024;
    T v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t q = from + threadIdx.x + 1024 * u;
        v[u] = q < to ? x[q] : T(0);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t q = from + threadIdx.x + 1024 * u;
        if (q < to) win[q % WL] = v[u];
    }
}

// fp atomic add in L2 (device-scope, relaxed); hardware fp32/fp64 atomics
// on coarse-grained device memory.
__device__ __forceinline__ void atomic_add(double* p, double v) {
    unsafeAtomicAdd(p, v);
}
__device__ __forceinline__ void atomic_add(float* p, float v) {
    unsafeAtomicAdd(p, v);
}

// y = alpha * s + beta * y; beta == 0 never reads y.
template <typename T>
__device__ __forceinline__ T axpby(T s, T alpha, T beta, const T* y) {
    return beta == T(0) ? alpha * s : alpha * s + beta * *y;
}

}  // namespace spmv
