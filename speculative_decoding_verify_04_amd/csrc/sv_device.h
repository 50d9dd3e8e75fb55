// Device-side helpers shared by the gfx950 kernels of libspecverify.
// Wave64 reductions, bf16 packing, and the MFMA operand vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ---- Wave-wide scans and reductions with DPP (data-parallel primitives).
// An inclusive scan over the 64 lanes takes seven DPP steps: row_shr 1, 2, 3
// (within rows of 16 lanes), row_shr 4 and 8 on the upper banks, then
// row_bcast 15 and 31 to carry between rows.  Lanes a step does not update
// receive the identity.  This runs at VALU speed; a scan built from
// ds_bpermute shuffles costs about three times as long on gfx950.  The order
// of the combinations is fixed, so results are bit-reproducible.
template <int CTRL, int ROW, int BANK>
__device__ __forceinline__ int dpp_i(int v, int identity) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW, BANK, true);
}
template <int CTRL, int ROW, int BANK>
__device__ __forceinline__ double dpp_d(double v) {
    const long long bits = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits), CTRL, ROW, BANK, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits >> 32), CTRL, ROW, BANK, true);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
template <int CTRL, int ROW, int BANK>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW, BANK, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, ROW, BANK, true);
    return (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo);
}

// Inclusive prefix sum across the wave in lane order (`lane` is unused; kept
// for call-site symmetry).
__device__ __forceinline__ double wave_incl_scan(double v, int /*lane*/) {
    double r = v + dpp_d<0x111, 0xF, 0xF>(v);
    r += dpp_d<0x112, 0xF, 0xF>(v);
    r += dpp_d<0x113, 0xF, 0xF>(v);
    r += dpp_d<0x114, 0xF, 0xE>(r);
    r += dpp_d<0x118, 0xF, 0xC>(r);
    r += dpp_d<0x142, 0xA, 0xF>(r);
    r += dpp_d<0x143, 0xC, 0xF>(r);
    return r;
}

__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
    int r = v + dpp_i<0x111, 0xF, 0xF>(v, 0);
    r += dpp_i<0x112, 0xF, 0xF>(v, 0);
    r += dpp_i<0x113, 0xF, 0xF>(v, 0);
    r += dpp_i<0x114, 0xF, 0xE>(r, 0);
    r += dpp_i<0x118, 0xF, 0xC>(r, 0);
    r += dpp_i<0x142, 0xA, 0xF>(r, 0);
    r += dpp_i<0x143, 0xC, 0xF>(r, 0);
    return r;
}

__device__ __forceinline__ unsigned long long wave_incl_scan(unsigned long long v, int /*lane*/) {
    unsigned long long r = v + dpp_u64<0x111, 0xF, 0xF>(v);
    r += dpp_u64<0x112, 0xF, 0xF>(v);
    r += dpp_u64<0x113, 0xF, 0xF>(v);
    r += dpp_u64<0x114, 0xF, 0xE>(r);
    r += dpp_u64<0x118, 0xF, 0xC>(r);
    r += dpp_u64<0x142, 0xA, 0xF>(r);
    r += dpp_u64<0x143, 0xC, 0xF>(r);
    return r;
}

// Value of lane 63 in every lane (a uniform result).
__device__ __forceinline__ double lane63(double v) {
    const long long bits = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(bits), 63);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(bits >> 32), 63);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

__device__ __forceinline__ double wave_sum(double v) { return lane63(wave_incl_scan(v, 0)); }

__device__ __forceinline__ int wave_sum(int v) {
    return __builtin_amdgcn_readlane(wave_incl_scan(v, 0), 63);
}

__device__ __forceinline__ float wave_sum(float v) {
    float r = v + __int_as_float(dpp_i<0x111, 0xF, 0xF>(__float_as_int(v), 0));
    r += __int_as_float(dpp_i<0x112, 0xF, 0xF>(__float_as_int(v), 0));
    r += __int_as_float(dpp_i<0x113, 0xF, 0xF>(__float_as_int(v), 0));
    r += __int_as_float(dpp_i<0x114, 0xF, 0xE>(__float_as_int(r), 0));
    r += __int_as_float(dpp_i<0x118, 0xF, 0xC>(__float_as_int(r), 0));
    r += __int_as_float(dpp_i<0x142, 0xA, 0xF>(__float_as_int(r), 0));
    r += __int_as_float(dpp_i<0x143, 0xC, 0xF>(__float_as_int(r), 0));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 63));
}

__device__ __forceinline__ float wave_max(float v) {
    const int ninf = __float_as_int(-INFINITY);
    float r = fmaxf(v, __int_as_float(dpp_i<0x111, 0xF, 0xF>(__float_as_int(v), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x112, 0xF, 0xF>(__float_as_int(v), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x113, 0xF, 0xF>(__float_as_int(v), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x114, 0xF, 0xE>(__float_as_int(r), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x118, 0xF, 0xC>(__float_as_int(r), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x142, 0xA, 0xF>(__float_as_int(r), ninf)));
    r = fmaxf(r, __int_as_float(dpp_i<0x143, 0xC, 0xF>(__float_as_int(r), ninf)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 63));
}

// Block-wide reductions for blockDim.x == NT (multiple of 64).  `red` is LDS
// scratch of at least NT/64 elements.  Every thread gets the result.  The
// combination order is fixed, so results are bit-reproducible.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

template <int NT>
__device__ __forceinline__ double block_sum(double v, double* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    double r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r += red[i];
    return r;
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    int r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r += red[i];
    return r;
}

// Workgroups are handed to the 8 XCDs of an MI355X round-robin by linear id.
// xcd_remap(L, n) returns a logical index such that logical indices
// [k*(n/8), (k+1)*(n/8)) all run on XCD k: consecutive logical blocks share an
// L2.  n must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int L, int n) {
    return (L & 7) * (n >> 3) + (L >> 3);
}

// ---- Hand-off of data between workgroups of one kernel.
// Data that another workgroup of the same launch reads is written with st_coh
// and read with ld_coh: relaxed atomics at agent scope, which the compiler
// emits as coherent (sc1) stores and loads.  The hand-off itself is an arrival
// counter (arrive_last).  No agent-scope fence is used: on gfx950 such a fence
// writes back and invalidates the whole L2 of the XCD, which costs far more
// than the few coherent accesses here.
template <typename T>
__device__ __forceinline__ void st_coh(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coh(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The relaxed hand-off below relies on gfx950's behaviour of sc1 accesses:
// coherent stores complete to the device-coherent level before s_waitcnt
// returns, and coherent loads do not hit stale lines in the reader's L2.  The
// HIP memory model alone would ask for a release on the counter and an
// acquire in the last arriver (SV_ARRIVE_RELEASE=1 builds that form; its
// measured cost is recorded with the design notes).  Other targets are
// refused at compile time rather than trusted.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "arrive_last's relaxed hand-off is argued for gfx950 only"
#endif
#ifndef SV_ARRIVE_RELEASE
#define SV_ARRIVE_RELEASE 0
#endif

// Called by all threads of a workgroup after its st_coh stores.  Waits until
// those stores have completed, counts the workgroup in *cnt, and returns true
// in the workgroup that arrives n-th (which also resets *cnt to 0 for the next
// launch).  That workgroup then sees every other workgroup's st_coh data
// through ld_coh.
__device__ __forceinline__ bool arrive_last(int* cnt, int n, int* flag_lds) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
#if SV_ARRIVE_RELEASE
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
#else
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#endif
        const int last = (old == n - 1) ? 1 : 0;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_lds = last;
    }
    __syncthreads();
    return *flag_lds != 0;
}

// Record the first device-side data error (0 = none).
__device__ __forceinline__ void set_status(int32_t* status, int code) {
    if (status) atomicCAS(status, 0, code);
}

}  // namespace sv
