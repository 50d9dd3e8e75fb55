// Target attention for the K+1 verify queries of every sequence, on gfx950.
//
// Method: "Accelerating Large Language Model Decoding with Speculative
// Sampling", section "Conditional scoring" (one target call scores all drafted
// positions; attention reads the whole KV cache and its cost does not grow with
// K); sequences keep ragged, unpadded lengths (BASS and EMS-SD abstracts); a
// prompt prefix shared by all sequences is read once (bifurcated-attention
// abstract: a GEMM over the shared prefill KV plus one over per-sample KV,
// exact result).
//
// Work decomposition (split-K over keys, flash-decoding style):
//   decode_bf16_kernel  one workgroup per work item (sequence b, chunk c, kv
//       head g).  The keys of sequence b are its L_b cached rows followed by
//       its K+1 new rows; each sequence is cut into chunks of at most
//       `lambda` 16-key slices, lambda chosen so that all work items fit in
//       one resident wave of workgroups.  Each of the 4 waves takes every 4th
//       slice; S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K rows go straight
//       from HBM into A-operand registers), an fp32 online softmax per query
//       column, and O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 (V is
//       transposed through LDS with ds_read_b64_tr_b16).  The query columns
//       of a kv head are its G = Hq/Hkv heads times the K+1 queries, in
//       16-wide tiles.  The last chunk of each (sequence, kv head) to finish
//       merges all partials (log-sum-exp) and writes the output rows; the
//       hand-off uses coherent stores/loads and an arrival counter, no cache
//       flush.
//   prefix_dma_kernel (D = 128) / prefix_bf16_kernel (D = 64)  one
//       workgroup per (prefix chunk, kv head, column group): every query
//       column of every sequence against one 128-key LDS tile at a time, so
//       the shared prefix is read from HBM once; the D = 128 form fills its
//       two tile buffers with direct global-to-LDS loads.
//   attn_f32_kernel  fp32 VALU path (small head dims, fp32 inputs).
//   merge_kernel  log-sum-exp merge of the fp32 path's partials.
// Scores are kept in the log2 domain (scale * log2(e) folded into S).
#include <stdlib.h>

#include <algorithm>
#include <vector>
#include <type_traits>

#include <hip/hip_ext.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kMergeMax = 1024;  // parts (prefix chunks + workgroups) merged per segment
constexpr int kMergeLds = 1536;  // (part, column) weights of a merge staged in LDS at a time

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const uint16_t* k_prefix;
    const uint16_t* v_prefix;
    const float* qf;
    const float* kcf;
    const float* vcf;
    const float* knf;
    const float* vnf;
    const float* kpf;
    const float* vpf;
    const int64_t* kv_start;
    const int32_t* kv_len;
    void* out;
    int32_t* status;
    float* part_o;     // bf16 path [slots][D][CPG]; fp32 path [slots][Hkv][CPG][D]
    float2* part_ml;   // bf16 path [slots][CPG]; fp32 path [slots][Hkv][CPG]  (m in log2 units, l)
    int* seq_base;     // [B] first slot of sequence b (fp32 path)
    int* merge_cnt;    // [B][Hkv] arrival counters of the fused merge (bf16 path)
    float* pre_o;      // [prefix_slots][Hkv][NC][D]
    float2* pre_ml;    // [prefix_slots][Hkv][NC]
    const int32_t* cu_q;  // [B+1] first query row of each sequence (ragged K_b), or null
    int rows;             // query rows in all: cu_q[B], or B*(K+1)
    int B, K, Hq, Hkv, G, CPG, NC, D, chunk, prefix_chunk, prefix_len, prefix_slots, slots;
    int lambda;        // bf16 path: 16-key slices per work item at most
    int bf16;
    int xcd;           // decode kernel: deal contiguous work items to each XCD
    float scale_log2;
};

// The decode kernel's work plan for up to kPlanB sequences, made on the host
// from the host length bound and passed in the kernel arguments: a workgroup
// finds its (sequence, chunk, kv head) without reading device memory.
constexpr int kPlanB = kAttnPlanB;
struct DecPlan {
    int nb;                    // B when the plan is valid; 0: find the plan on the device
    int q[kPlanB + 1];         // q[b] = first chunk of sequence b; q[nb] = chunks in all
                               // (even split: q[b] = items of the sequences before b)
    int s[kPlanB];             // 16-key slices (even split: 32-key items) of sequence b
                               // for its host bound
    int row0[kPlanB + 1];      // first query row of sequence b; row0[nb] = query rows
    int W;                     // even split: item ranges per kv head (0: per-sequence chunks)
    long long N;               // even split: 32-key items of all sequences (one kv head)
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Query rows of sequence b: cu_q[b] .. cu_q[b+1]-1 (K_b + 1 rows, K_b <= K), or
// b*(K+1) .. b*(K+1)+K without cu_q.  Its new K/V rows have the same indices.
__device__ __forceinline__ int seq_q0(const AttnParams& p, int b) {
    return p.cu_q ? p.cu_q[b] : b * (p.K + 1);
}
__device__ __forceinline__ int seq_k1(const AttnParams& p, int b) {
    return p.cu_q ? min(max(p.cu_q[b + 1] - p.cu_q[b], 1), p.K + 1) : p.K + 1;
}

// Work item x (a global chunk index) -> (sequence, chunk within it), computed by
// wave 0 from the device lengths; writes s_b = -1 when x is past the last chunk.
__device__ void find_sequence(const AttnParams& p, int x, int g, int* s_b, int* s_c) {
    const int lane = threadIdx.x & 63;
    int run = 0, fb = -1, fc = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        int n = 0;
        if (b < p.B) {
            int L = p.kv_len[b];
            if (L < 0) {
                if (x == 0 && g == 0) set_status(p.status, 3);
                L = 0;
            }
            n = ceil_div(L + seq_k1(p, b), p.chunk);
        }
        const int inc = wave_incl_scan(n, lane) + run;
        const int excl = inc - n;
        if (b < p.B && x >= excl && x < inc) { fb = b; fc = x - excl; }
        run = __shfl(inc, 63, 64);
    }
    // fold the owning lane's answer into lane 0
    unsigned long long own = __ballot(fb >= 0);
    int src = own ? __ffsll(own) - 1 : 0;
    fb = __shfl(fb, src, 64);
    fc = __shfl(fc, src, 64);
    if (lane == 0) {
        *s_b = own ? fb : -1;
        *s_c = fc;
        if (x == 0 && g == 0 && run > p.slots) set_status(p.status, 3);
    }
}


#ifndef SV_NCT1_WAVES
#define SV_NCT1_WAVES 3
#endif

// ---------------------------------------------------------------- decode (bf16)
//
// Split-K over keys with one work item per workgroup.  The keys of sequence b
// are its L_b cached rows followed by its K+1 new rows: S_b = ceil((L_b+K+1)/16)
// slices of 16 keys.  With a slice budget `lambda` chosen on the host (the
// smallest one for which the work items fit in one resident wave of
// workgroups), sequence b is cut into q_b = ceil(S_b / lambda) chunks of
// equal size (+-1 slice), and work item (b, chunk c, kv head g) is workgroup
// Hkv * (q_0 + .. + q_{b-1}) + c * Hkv + g.  The kv head varies fastest, so
// workgroups running side by side read the same cache rows for all heads
// (whole DRAM rows instead of scattered 256-byte pieces).  Each of the 4
// waves takes every 4th slice of the chunk and keeps the next one in flight.
// At the end the workgroup combines its waves and writes one partial (m, l, o);
// the last chunk of a (sequence, head) to arrive merges all of them and the
// shared-prefix partials of the prefix kernel, and writes the output rows.

constexpr int kSkMaxB = 2048;        // sequences per call on the bf16 path
constexpr int kLambdaMax = 192;      // 16-key slices per work item at most (long problems)
constexpr int kLambdaMin = 12;       // 16-key slices per work item at least
constexpr int kSkMaxKeys = 1 << 25;  // keys per sequence on the bf16 path

typedef short v4s_t __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i supplies the address of 4 consecutive b16 values that form
// row i/4, columns 4*(i%4) .. 4*(i%4)+3 of a 4 x 16 tile; lane n receives
// column n of that tile (rows 0..3).
__device__ __forceinline__ shortx4 lds_read_tr16(const uint16_t* p) {
    v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(const_cast<uint16_t*>(p)));
    return shortx4{r[0], r[1], r[2], r[3]};
}

// Max and sum over the lanes {l, l^16, l^32, l^48} (the four key groups of one
// query column) with the gfx950 lane swaps: v_permlane16_swap exchanges rows 0
// and 1, 2 and 3 (16 lanes each) between its two operands, v_permlane32_swap
// the two halves of the wave; with both operands equal to x, the two results
// hold x and its partner's value on every lane.  VALU only, no LDS traffic.
__device__ __forceinline__ float colmax4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colsum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int NCT>
struct DecLds {
    static constexpr int VP = D + 4;   // V slice pitch (bf16)
    static constexpr int OP = 20;      // column pitch of the wave-combine buffer (floats)
    union {
        uint16_t vs[4][16][VP];
        struct {
            float o[4][D / 2][OP];     // [wave][d within the half][column]
            float m[4][16];
            float l[4][16];
        } red;
        struct {
            float2 ml[kMergeLds];      // (m, l) of (part, column) pairs of a column group
            float w[kMergeLds];        // their merge weights
        } mrg;
    };
    uint16_t qs[NCT * 16][D + 8];      // the work item's query columns (B operand source)
    int Q[kSkMaxB + 1];                // Q[b] = q_0 + .. + q_{b-1}
    int L;                             // kv_len of this workgroup's sequence
    int k1;                            // its query rows (K_b + 1)
    int q0;                            // its first query row
    long long kv0;                     // kv_start of this workgroup's sequence
    int flag;
};

// LDS of the column-wave form: the query tiles (read into registers at the
// start), the device plan's prefix sums (prologue) and the merge's weights
// (end) are never live at once.
template <int D, int NCT>
struct DecLdsCol {
    static constexpr int VP = D + 4;
    union {
        uint16_t qs[NCT * 16][D + 8];
        int Q[kSkMaxB + 1];
        struct {
            float2 ml[kMergeLds];
            float w[kMergeLds];
        } mrg;
    };
    int L;
    int k1;
    int q0;
    long long kv0;
    int flag;
};

// Online softmax of one 16-column tile's scores on one 16-key slice (S^T tile
// `acc`: keys k0 + kg*4 + ee of column col16; keys at or past `limt` masked
// unless `full`) and O^T += V^T P^T with the slice's V^T operands `va`.
template <int DT>
__device__ __forceinline__ void col_tile_update(int kg, float scale_log2, int k0, bool full, int limt,
                                                const floatx4& acc, const shortx4 (&va)[DT], float& mr,
                                                float& lr, floatx4 (&ot)[DT]) {
    float s[4];
    float mt = -INFINITY;
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
        const int tt = k0 + kg * 4 + ee;
        s[ee] = (full || tt < limt) ? acc[ee] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, s[ee]);
    }
    mt = colmax4(mt);
    const float mnew = fmaxf(mr, mt);
    // the running max of no column of the tile grew: alpha would be exactly 1
    // on every lane, so the rescale of O is skipped (most slices after the
    // first few)
    const bool grew = __ballot(mt > mr) != 0;
    float alpha = 1.0f;
    shortx4 pb;
    if (mnew == -INFINITY) {
        pb = shortx4{0, 0, 0, 0};
    } else {
        if (grew) alpha = __builtin_amdgcn_exp2f(mr - mnew);
        float pe[4];
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) pe[ee] = __builtin_amdgcn_exp2f(s[ee] - mnew);
        lr = lr * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
        mr = mnew;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) pb[ee] = static_cast<short>(f32_to_bf16(pe[ee]));
    }
    if (grew) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ot[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        ot[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], pb, ot[dt], 0, 0, 0);
}

// Merge of the partials of (sequence, kv head g) when no prefix part is
// involved and every value a thread needs fits in registers (UP (d, column)
// pairs per thread, PMAX parts): the partial loads are issued before the
// (m, l) loads, so both travel in the same round trip; the weights are formed
// in LDS; fixed order, as in dec_merge.
// With np > 0 the first np parts are the shared prefix's chunk partials of
// sequence b (written by the prefix kernel), the rest at first_slot + (j -
// np)*stride.
template <int D, int UP, int PMAX, typename MRG>
__device__ __forceinline__ void merge_in_registers(const AttnParams& p, MRG& M, int b, int g, int first_slot,
                                                   int stride, int np, int nparts, int nc, int qrow0,
                                                   int k1) {
    const int tid = threadIdx.x;
    const int CPG = p.CPG, npairs = nc * D;
    const size_t pre_col0 = static_cast<size_t>(g) * p.NC + static_cast<size_t>(b) * CPG;
    float ov[PMAX][UP];
    int off[UP], poff[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) {
        const int pq = min(tid + u * kThreads, npairs - 1);
        off[u] = (pq / nc) * CPG + pq % nc;
        poff[u] = (pq % nc) * D + pq / nc;  // prefix partials: [chunk][Hkv][NC][D]
    }
#pragma unroll
    for (int jj = 0; jj < PMAX; ++jj) {
        const int j = min(jj, nparts - 1);  // past the end: re-read the last part
        if (j < np) {
            const float* pb = p.pre_o + (static_cast<size_t>(j) * p.Hkv * p.NC + pre_col0) * D;
#pragma unroll
            for (int u = 0; u < UP; ++u) ov[jj][u] = pb[poff[u]];
        } else {
            const float* pb =
                p.part_o + (static_cast<size_t>(first_slot) + static_cast<size_t>(j - np) * stride) * D * CPG;
#pragma unroll
            for (int u = 0; u < UP; ++u) ov[jj][u] = ld_coh(pb + off[u]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < nparts * nc; idx += kThreads) {
        const int j = idx / nc, col = idx % nc;
        if (j < np) {
            M.ml[idx] = p.pre_ml[static_cast<size_t>(j) * p.Hkv * p.NC + pre_col0 + col];
        } else {
            const unsigned long long u = ld_coh(reinterpret_cast<const unsigned long long*>(
                p.part_ml + (static_cast<size_t>(first_slot) + static_cast<size_t>(j - np) * stride) * CPG + col));
            M.ml[idx] = make_float2(__uint_as_float(static_cast<unsigned>(u)),
                                    __uint_as_float(static_cast<unsigned>(u >> 32)));
        }
    }
    __syncthreads();
    for (int cl = tid; cl < nc; cl += kThreads) {
        float ms = -INFINITY;
        for (int j = 0; j < nparts; ++j) ms = fmaxf(ms, M.ml[j * nc + cl].x);
        float l = 0.0f;
        for (int j = 0; j < nparts; ++j) {
            const float2 v = M.ml[j * nc + cl];
            const float f = (v.x == -INFINITY) ? 0.0f : exp2f(v.x - ms);
            M.w[j * nc + cl] = f;
            l += v.y * f;
        }
        const float inv = 1.0f / l;
        for (int j = 0; j < nparts; ++j) M.w[j * nc + cl] *= inv;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < UP; ++u) {
        const int pq = tid + u * kThreads;
        if (pq >= npairs) continue;
        const int cl = pq % nc, d = pq / nc;
        float acc = 0.0f;
#pragma unroll
        for (int jj = 0; jj < PMAX; ++jj)
            if (jj < nparts) acc += ov[jj][u] * M.w[jj * nc + cl];
        const int hh = cl / k1, j = cl % k1;
        const size_t oi = (static_cast<size_t>(qrow0 + j) * p.Hq + g * p.G + hh) * D + d;
        static_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(acc);
    }
}

// Merge every part of (sequence b, kv head g) -- the prefix chunks first, then
// its q_b chunks in order, at partial slots first_slot + j*stride -- and write
// the output rows qrow0+j (j < k1) of heads g*G + hh.  When every value a
// thread needs fits in registers, one round trip (merge_in_registers); else
// two: the (m, l) of every (part, column) into LDS and
// the per-column weights, then every o value weighted, with the loads of up
// to 4 columns x 8 parts in flight per thread.  Fixed order: bit-reproducible.
template <int D, int NCT, typename MRG>
__device__ __forceinline__ void dec_merge(const AttnParams& p, MRG& M, int b, int g, int first_slot, int stride, int qb,
                          int qrow0, int k1) {
    const int tid = threadIdx.x;
    const int np = p.prefix_slots;
    const int nparts = np + qb;
    const int CPG = p.CPG;
    const int ncols = p.G * k1;  // the sequence's columns (hh * k1 + j)
    const size_t pre_col0 = static_cast<size_t>(g) * p.NC + static_cast<size_t>(b) * CPG;
    auto slot_of = [&](int j) {  // partial slot of stream part j >= np
        return static_cast<size_t>(first_slot) + static_cast<size_t>(j - np) * stride;
    };
    constexpr int cap = static_cast<int>(sizeof(M.w) / sizeof(M.w[0]));  // (part, column) pairs in LDS
    const int group = max(1, min(ncols, cap / nparts));
    if (group == ncols) {
        // every partial value a thread needs fits in registers: one round trip
        const int npairs = ncols * D;
        if (np == 0 && nparts <= 8 && npairs <= 4 * kThreads) {
            merge_in_registers<D, 4, 8>(p, M, b, g, first_slot, stride, 0, nparts, ncols, qrow0, k1);
            return;
        }
        // with a shared prefix (its chunks, then the sequence's own parts)
        if (np > 0 && nparts <= 12 && npairs <= 3 * kThreads) {
            merge_in_registers<D, 3, 12>(p, M, b, g, first_slot, stride, np, nparts, ncols, qrow0, k1);
            return;
        }
        // (the wider forms only where the kernel's loop already needs more
        // registers than they do: the one-tile kernel stays at 4 workgroups
        // per CU)
        if constexpr (NCT > 1) {
            if (np == 0 && nparts <= 4 && npairs <= 8 * kThreads) {
                merge_in_registers<D, 8, 4>(p, M, b, g, first_slot, stride, 0, nparts, ncols, qrow0, k1);
                return;
            }
            if (np == 0 && nparts <= 2 && npairs <= 20 * kThreads) {
                merge_in_registers<D, 20, 2>(p, M, b, g, first_slot, stride, 0, nparts, ncols, qrow0, k1);
                return;
            }
        }
    }
    for (int c0 = 0; c0 < ncols; c0 += group) {
        const int nc = min(group, ncols - c0);
        __syncthreads();
        for (int idx = tid; idx < nparts * nc; idx += kThreads) {
            const int j = idx / nc, col = c0 + idx % nc;
            float2 v;
            if (j < np) {
                v = p.pre_ml[static_cast<size_t>(j) * p.Hkv * p.NC + pre_col0 + col];
            } else {
                const unsigned long long u =
                    ld_coh(reinterpret_cast<const unsigned long long*>(p.part_ml + slot_of(j) * CPG + col));
                v = make_float2(__uint_as_float(static_cast<unsigned>(u)),
                                __uint_as_float(static_cast<unsigned>(u >> 32)));
            }
            M.ml[idx] = v;
        }
        __syncthreads();
        for (int cl = tid; cl < nc; cl += kThreads) {
            float ms = -INFINITY;
            for (int j = 0; j < nparts; ++j) ms = fmaxf(ms, M.ml[j * nc + cl].x);
            float l = 0.0f;
            for (int j = 0; j < nparts; ++j) {
                const float2 v = M.ml[j * nc + cl];
                const float f = (v.x == -INFINITY) ? 0.0f : exp2f(v.x - ms);
                M.w[j * nc + cl] = f;
                l += v.y * f;
            }
            const float inv = 1.0f / l;
            for (int j = 0; j < nparts; ++j) M.w[j * nc + cl] *= inv;
        }
        __syncthreads();
        const int npairs = nc * D;
        for (int q0 = tid; q0 < npairs; q0 += 4 * kThreads) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            int off[4];  // element offset of pair u inside one part ([d][column] layout)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pq = min(q0 + u * kThreads, npairs - 1);
                off[u] = (pq / nc) * CPG + c0 + pq % nc;
            }
            for (int j0 = 0; j0 < nparts; j0 += 8) {
                float ov[8][4];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int j = min(j0 + jj, nparts - 1);  // past the end: re-read the last part
                    // the part's base is uniform over the workgroup
                    const float* pb = (j < np) ? nullptr : p.part_o + slot_of(j) * D * CPG;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (j < np) {
                            const int pq = min(q0 + u * kThreads, npairs - 1);
                            ov[jj][u] = p.pre_o[(static_cast<size_t>(j) * p.Hkv * p.NC + pre_col0 + c0 +
                                                 pq % nc) * D + pq / nc];
                        } else {
                            ov[jj][u] = ld_coh(pb + off[u]);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int cl = min(q0 + u * kThreads, npairs - 1) % nc;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        if (j0 + jj < nparts) acc[u] += ov[jj][u] * M.w[(j0 + jj) * nc + cl];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pq = q0 + u * kThreads;
                if (pq >= npairs) continue;
                const int cl = pq % nc, d = pq / nc, col = c0 + cl;
                const int hh = col / k1, j = col % k1;
                const size_t oi = (static_cast<size_t>(qrow0 + j) * p.Hq + g * p.G + hh) * D + d;
                static_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(acc[u]);
            }
        }
    }
}

// Position of the 16-byte chunk c of a 128-wide bf16 row r in LDS: c ^ swz(r).
// The 16-byte K reads of 16 consecutive rows and the transposed 8-byte V reads
// of 16 rows x 2 chunks then fall on distinct LDS banks.
__device__ __forceinline__ int prefix_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// One 16-key slice of K and V for the whole workgroup (column-wave form),
// filled by direct global-to-LDS loads (D = 128: rows of 16 chunks, chunk c
// of row r at c ^ prefix_swz(r)).  The kernel holds six as separate LDS
// objects, so the compiler can tell reads of one from direct loads still
// landing in the others.
struct DecColSlot {
    uint4 k[16 * 16];
    uint4 v[16 * 16];
};

// K and V of one 16-key slice held in registers.
template <int D>
struct Slice {
    bf16x8 k[D / 32];
    uint4 v[16 * (D / 8) / 64];
};

// MODE 0: each wave takes every 4th slice of the item for all NCT column
// tiles and keeps its next slice in registers.  MODE 2 (D = 128, NCT 2..4):
// column waves -- wave w < NCT takes column tile w over every slice of the
// item, so it holds one tile's accumulators instead of NCT (the multi-tile
// form of mode 0 runs one wave per SIMD); the slices pass through a six-slot
// LDS ring that all four waves fill with direct loads, one barrier per
// slice, and no wave combine is needed.
template <int D, int NCT, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NCT == 1 ? SV_NCT1_WAVES : (MODE == 2 ? 2 : 1))))
void decode_bf16_kernel(AttnParams p, DecPlan plan) {
    static_assert(MODE == 0 || (MODE == 2 && D == 128), "the ring layout is for 128-wide heads");
    constexpr int KK = D / 32;   // 16x16x32 steps over the head dim
    constexpr int DT = D / 16;   // 16-wide head-dim tiles of the PV product
    constexpr int VCH = D / 8;   // 16-byte chunks per K/V row
    constexpr int VLD = 16 * VCH / 64;  // 16-byte V loads per lane per slice
    constexpr int VP = DecLds<D, NCT>::VP;
    constexpr int NPRO = kSkMaxB / kThreads;
    using LdsT = typename std::conditional<MODE == 2, DecLdsCol<D, NCT>, DecLds<D, NCT>>::type;
    __shared__ LdsT S;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col16 = lane & 15, kg = lane >> 4;
    const int lambda = p.lambda;
    // with p.xcd the grid is a multiple of 8 and XCD x (which runs workgroups
    // x, x+8, ...) gets the contiguous work items [x*n/8, (x+1)*n/8)
    const int id = p.xcd ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;

    int b, qb, c, g, first_slot, L, k1, q0, Sb;
    long long kv0;
    if (plan.nb > 0) {
        // ---- host plan: b = the number of sequences whose chunks all precede
        // this workgroup's chunk (a ballot over the sequences)
        const int cidx = id / p.Hkv;
        int cnt = 0;
        for (int b0 = 0; b0 < plan.nb; b0 += 64) {
            const int bb = b0 + lane;
            cnt += __popcll(__ballot((bb < plan.nb) && (plan.q[bb + 1] <= cidx)));
        }
        b = __builtin_amdgcn_readfirstlane(cnt);
        if (b >= plan.nb) return;  // past the last work item
        const int qlo = plan.q[b];
        qb = plan.q[b + 1] - qlo;
        c = cidx - qlo;
        g = id - cidx * p.Hkv;
        first_slot = p.Hkv * qlo;
        Sb = plan.s[b];
        q0 = plan.row0[b];
        k1 = plan.row0[b + 1] - q0;
        // the sequence's device data, one round trip; every workgroup of a
        // sequence takes the same decision, so a bad sequence arrives nowhere
        L = p.kv_len[b];
        kv0 = p.kv_start[b];
        bool bad = (L < 0) || (static_cast<long long>(L) + k1 > 16LL * Sb);
        if (p.cu_q) bad = bad || (p.cu_q[b] != q0) || (p.cu_q[b + 1] != q0 + k1);
        if (bad) {
            if (c == 0 && g == 0 && tid == 0) set_status(p.status, 3);
            return;
        }
    } else {
        // ---- chunks per sequence from the device lengths and their prefix
        // sum (one round trip), then a binary search
        int Lr[NPRO], Kr[NPRO];
        long long Sr[NPRO];
#pragma unroll
        for (int u = 0; u < NPRO; ++u) {
            const int bb = tid + u * kThreads;
            Lr[u] = 0;
            Sr[u] = 0;
            Kr[u] = p.K + 1;
            if (bb < p.B) {
                Lr[u] = p.kv_len[bb];
                Sr[u] = p.kv_start[bb];
                if (p.cu_q) Kr[u] = p.cu_q[bb + 1] - p.cu_q[bb];
            }
        }
#pragma unroll
        for (int u = 0; u < NPRO; ++u) {
            const int bb = tid + u * kThreads;
            if (bb < p.B) {
                if (Lr[u] < 0) {
                    if (id == 0) set_status(p.status, 3);
                    Lr[u] = 0;
                }
                Lr[u] = min(Lr[u], kSkMaxKeys);
                if (Kr[u] < 1 || Kr[u] > p.K + 1) {  // device offsets disagree with the host's
                    if (id == 0) set_status(p.status, 3);
                    Kr[u] = min(max(Kr[u], 1), p.K + 1);
                }
                S.Q[bb + 1] = ceil_div(ceil_div(Lr[u] + Kr[u], 16), lambda);
            }
        }
        __syncthreads();
        if (w == 0) {
            int run = 0, qmax = 0;
            for (int b0 = 0; b0 < p.B; b0 += 64) {
                const int v = (b0 + lane < p.B) ? S.Q[b0 + lane + 1] : 0;
                qmax = max(qmax, v);
                const int inc = wave_incl_scan(v, lane) + run;
                if (b0 + lane < p.B) S.Q[b0 + lane + 1] = inc;
                run = __shfl(inc, 63, 64);
            }
            qmax = static_cast<int>(wave_max(static_cast<float>(qmax)));  // exact below 2^24
            if (lane == 0) {
                S.Q[0] = 0;
                S.flag = qmax;
            }
        }
        __syncthreads();
        // Device lengths above the host bound would need more work items than
        // the launch has, or more chunks of one sequence than the merge takes:
        // every workgroup sees the same totals and leaves.
        const long long items = static_cast<long long>(p.Hkv) * S.Q[p.B];
        if (items > static_cast<long long>(gridDim.x) || S.flag + p.prefix_slots > kMergeMax) {
            if (id == 0 && tid == 0) set_status(p.status, 3);
            return;
        }
        if (id >= items) return;
        {
            int lo = 0, hi = p.B - 1;  // largest b with Hkv * Q[b] <= id
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (p.Hkv * S.Q[mid] <= id) lo = mid; else hi = mid - 1;
            }
            b = __builtin_amdgcn_readfirstlane(lo);
        }
        first_slot = p.Hkv * S.Q[b];
        qb = S.Q[b + 1] - S.Q[b];
        c = (id - first_slot) / p.Hkv;
        g = (id - first_slot) % p.Hkv;
        __syncthreads();  // S.flag is reused by the merge hand-off
#pragma unroll
        for (int u = 0; u < NPRO; ++u) {
            if (tid + u * kThreads == b) {
                S.L = Lr[u];
                S.kv0 = Sr[u];
                S.k1 = Kr[u];
                S.q0 = p.cu_q ? p.cu_q[b] : b * (p.K + 1);
            }
        }
        __syncthreads();
        L = __builtin_amdgcn_readfirstlane(S.L);
        k1 = __builtin_amdgcn_readfirstlane(S.k1);  // K_b + 1 query rows
        q0 = __builtin_amdgcn_readfirstlane(S.q0);  // the first of them
        kv0 = S.kv0;
    }
    // the qb chunks of the sequence share its slices for the device length
    // (a host bound above it leaves no masked slices, at most empty chunks)
    Sb = ceil_div(L + k1, 16);
    const int ncols = p.G * k1;
    const int T = L + k1;       // keys of the sequence (on the device)
    const int sl_lo = static_cast<int>(static_cast<long long>(c) * Sb / qb);
    const int sl_hi = static_cast<int>(static_cast<long long>(c + 1) * Sb / qb);

    const int rs = p.Hkv * D;  // elements per cache row
    const size_t head = static_cast<size_t>(g) * D;

    // Slice of keys [k0, k0+16) into registers.  Every lane addresses its own
    // row: cache rows for keys < L, new rows after them; keys past the last
    // one are clamped to it (and masked).
    auto row = [&](int tt, const uint16_t* cache, const uint16_t* fresh) __attribute__((always_inline)) -> const uint16_t* {
        tt = min(tt, T - 1);
        return (tt < L) ? cache + static_cast<size_t>(kv0 + tt) * rs + head
                        : fresh + static_cast<size_t>(q0 + (tt - L)) * rs + head;
    };
    auto load_slice = [&](Slice<D>& sl, int k0) __attribute__((always_inline)) {
        const uint16_t* kp = row(k0 + col16, p.k_cache, p.k_new) + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sl.k[kk] = *reinterpret_cast<const bf16x8*>(kp + 32 * kk);
#pragma unroll
        for (int q = 0; q < VLD; ++q)
            sl.v[q] = *reinterpret_cast<const uint4*>(row(k0 + (q * 64 + lane) / VCH, p.v_cache, p.v_new) +
                                                      ((q * 64 + lane) % VCH) * 8);
    };

    Slice<D> sl;
    if constexpr (MODE == 0) {
        if (sl_lo + w < sl_hi) load_slice(sl, (sl_lo + w) * 16);
    }
    // (the sequence's length and first cache row as wave-uniform scalars, and
    // the row chosen by selects: the direct loads then wait for nothing)
    const int Lu = __builtin_amdgcn_readfirstlane(L);
    const long long kv0u = static_cast<long long>(
        (static_cast<unsigned long long>(static_cast<unsigned>(__builtin_amdgcn_readfirstlane(
             static_cast<int>(kv0 >> 32))))
         << 32) |
        static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(kv0))));
    const uint16_t* const kc = p.k_cache;  // (kernel arguments as scalars, not loads)
    const uint16_t* const vc = p.v_cache;
    const uint16_t* const kn = p.k_new;
    const uint16_t* const vn = p.v_new;
    auto row_sel = [&](int tt, const uint16_t* cache, const uint16_t* fresh) __attribute__((always_inline)) -> const uint16_t* {
        tt = min(tt, T - 1);
        const bool in_cache = tt < Lu;
        const long long ri = in_cache ? kv0u + tt : static_cast<long long>(q0 + (tt - Lu));
        return (in_cache ? cache : fresh) + static_cast<size_t>(ri) * rs + head;
    };
    // column waves: every slice of the item; wave w loads blocks 2w, 2w+1
    // (waves 0, 1: K rows 0-7, 8-15; waves 2, 3: the same V rows)
    const int nslc = sl_hi - sl_lo;
    const bool cisv = w >= 2;
    const int cbb0 = 2 * (w & 1);
    // row within the slice and element offset of this lane's 16 bytes, per block
    const int cr0 = cbb0 * 4 + (lane >> 4), cr1 = cr0 + 4;
    const int cp0 = (lane & 15) ^ prefix_swz(cr0), cp1 = (lane & 15) ^ prefix_swz(cr1);
    const int coff0 = cr0 * rs + static_cast<int>(head) + cp0 * 8;
    const int coff1 = cr1 * rs + static_cast<int>(head) + cp1 * 8;
    auto issue_c = [&](int j, DecColSlot& R) __attribute__((always_inline)) {
        const int k0 = (sl_lo + j) * 16;
        if (k0 + 15 < Lu) {  // uniform: every row of the slice is a cache row
            const size_t base = static_cast<size_t>(kv0u + k0) * rs;
            const uint16_t* src0 = (cisv ? vc : kc) + base + coff0;
            const uint16_t* src1 = (cisv ? vc : kc) + base + coff1;
            __builtin_amdgcn_global_load_lds(src0, (cisv ? R.v : R.k) + cbb0 * 64, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(src1, (cisv ? R.v : R.k) + cbb0 * 64 + 64, 16, 0, 0);
        } else {
            const uint16_t* src0 = row_sel(k0 + cr0, cisv ? vc : kc, cisv ? vn : kn) + cp0 * 8;
            const uint16_t* src1 = row_sel(k0 + cr1, cisv ? vc : kc, cisv ? vn : kn) + cp1 * 8;
            __builtin_amdgcn_global_load_lds(src0, (cisv ? R.v : R.k) + cbb0 * 64, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(src1, (cisv ? R.v : R.k) + cbb0 * 64 + 64, 16, 0, 0);
        }
    };
    // six slots: slice j in slot j mod 6, five slices in flight
    __shared__ DecColSlot C0, C1, C2, C3, C4, C5;  // referenced only when MODE == 2
    if constexpr (MODE == 2) {
        if (nslc > 0) issue_c(0, C0);
        if (nslc > 1) issue_c(1, C1);
        if (nslc > 2) issue_c(2, C2);
        if (nslc > 3) issue_c(3, C3);
        if (nslc > 4) issue_c(4, C4);
    }

    // the work item's query columns -> LDS (zero rows for padding columns)
    for (int idx = tid; idx < NCT * 16 * VCH; idx += kThreads) {
        const int col = idx / VCH, ch = idx % VCH;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col < ncols) {
            const int hh = col / k1, j = col % k1;
            v = *reinterpret_cast<const uint4*>(
                p.q + (static_cast<size_t>(q0 + j) * p.Hq + g * p.G + hh) * D + ch * 8);
        }
        uint2* dst = reinterpret_cast<uint2*>(&S.qs[col][ch * 8]);
        dst[0] = make_uint2(v.x, v.y);
        dst[1] = make_uint2(v.z, v.w);
    }
    int lim[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = ct * 16 + col16;
        lim[ct] = (col < ncols) ? L + col % k1 + 1 : 0;
    }
    __syncthreads();

    floatx4 o[NCT][DT];
    float mrun[NCT], lrun[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        mrun[ct] = -INFINITY;
        lrun[ct] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[ct][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    auto tile_update = [&](int k0, bool full, int limt, const floatx4& acc, const shortx4 (&va)[DT],
                           float& mr, float& lr, floatx4 (&ot)[DT]) __attribute__((always_inline)) {
        col_tile_update<DT>(kg, p.scale_log2, k0, full, limt, acc, va, mr, lr, ot);
    };
    auto softmax_pv = [&](int k0, const floatx4 (&acc)[NCT], const shortx4 (&va)[DT]) __attribute__((always_inline)) {
        const bool full = k0 + 15 < L;  // no key of the slice is masked for any column
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) tile_update(k0, full, lim[ct], acc[ct], va, mrun[ct], lrun[ct], o[ct]);
    };

    // K operand of a ring slot: row col16, logical chunk kg + 4 kk, stored at
    // (kg ^ (sk & 3)) + 4 (kk ^ (sk >> 2)); V^T operand: row rv = kg*4 +
    // col16/4, logical chunk 2 dt + h (h = (col16 & 3) >> 1), 8-byte half
    // col16 & 1, stored at chunk 2 (dt ^ (sv >> 1)) + (h ^ (sv & 1))
    const int csk = prefix_swz(col16);
    const int ckcol = col16 * 16 + (kg ^ (csk & 3));
    const int csk2 = csk >> 2;
    const int crv = kg * 4 + (col16 >> 2);
    const int csv = prefix_swz(crv);
    const int csv1 = csv >> 1;
    const int cvcol = crv * D + 8 * (((col16 & 3) >> 1) ^ (csv & 1)) + 4 * (col16 & 1);
    // column waves: this wave's tile and its state
    float mcw = -INFINITY, lcw = 0.0f;
    floatx4 ocw[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ocw[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == 2) {
        const bool cw = w < NCT;  // uniform: this wave computes tile w
        const int colw = w * 16 + col16;
        const int limw = (cw && colw < ncols) ? L + colw % k1 + 1 : 0;
        bf16x8 qv[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qv[kk] = *reinterpret_cast<const bf16x8*>(&S.qs[(cw ? w : 0) * 16 + col16][kg * 8 + 32 * kk]);
        auto step_c = [&](int j, DecColSlot& R, DecColSlot& Rn) __attribute__((always_inline)) {
            // this wave's blocks of slice j are in when at most those of the
            // slices issued after it (j+1 .. j+4, two each) are in flight
            switch (min(4, nslc - 1 - j)) {
                case 4: __builtin_amdgcn_s_waitcnt(0x0F78); break;  // vmcnt(8)
                case 3: __builtin_amdgcn_s_waitcnt(0x0F76); break;  // vmcnt(6)
                case 2: __builtin_amdgcn_s_waitcnt(0x0F74); break;  // vmcnt(4)
                case 1: __builtin_amdgcn_s_waitcnt(0x0F72); break;  // vmcnt(2)
                default: __builtin_amdgcn_s_waitcnt(0x0F70); break; // vmcnt(0)
            }
            __syncthreads();  // every block of slice j is in R; slice j-1 (in Rn) is read
            if (j + 5 < nslc) issue_c(j + 5, Rn);
            if (cw) {
                const int k0 = (sl_lo + j) * 16;
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(R.k + ckcol + 4 * (kk ^ csk2));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[kk], acc, 0, 0, 0);
                }
                const uint16_t* vb = reinterpret_cast<const uint16_t*>(R.v);
                shortx4 va[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) va[dt] = lds_read_tr16(vb + cvcol + 16 * (dt ^ csv1));
                tile_update(k0, k0 + 15 < L, limw, acc, va, mcw, lcw, ocw);
            }
        };
        for (int j = 0; j < nslc; j += 6) {
            step_c(j, C0, C5);
            if (j + 1 < nslc) step_c(j + 1, C1, C0);
            if (j + 2 < nslc) step_c(j + 2, C2, C1);
            if (j + 3 < nslc) step_c(j + 3, C3, C2);
            if (j + 4 < nslc) step_c(j + 4, C4, C3);
            if (j + 5 < nslc) step_c(j + 5, C5, C4);
        }
    } else {
        uint16_t(*vs)[VP] = S.vs[w];
        // transposed-read address of this lane: row kg*4 + col16/4, column 4*(col16%4)
        const uint16_t* vt_base = &vs[kg * 4 + (col16 >> 2)][(col16 & 3) * 4];
        // Per slice: stage V in LDS, S^T = K Q^T, then reissue the slice
        // registers for the wave's next slice (in flight during the softmax
        // and the PV product).
        for (int si = sl_lo + w; si < sl_hi; si += 4) {
            const int k0 = si * 16;
#pragma unroll
            for (int q = 0; q < VLD; ++q) {
                uint2* dst = reinterpret_cast<uint2*>(&vs[(q * 64 + lane) / VCH][((q * 64 + lane) % VCH) * 8]);
                dst[0] = make_uint2(sl.v[q].x, sl.v[q].y);
                dst[1] = make_uint2(sl.v[q].z, sl.v[q].w);
            }
            floatx4 acc[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8 qop =
                        *reinterpret_cast<const bf16x8*>(&S.qs[ct * 16 + col16][kg * 8 + 32 * kk]);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl.k[kk], qop, acc[ct], 0, 0, 0);
                }
            }
            if (si + 4 < sl_hi) load_slice(sl, k0 + 64);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // V^T operands: lane (d = dt*16 + col16) gets keys kg*4 .. kg*4+3
            shortx4 va[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) va[dt] = lds_read_tr16(vt_base + dt * 16);
            softmax_pv(k0, acc, va);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        lrun[ct] = colsum4(lrun[ct]);
    }

    // combine the 4 waves (fixed order) in two halves of the head dim; the
    // partial of work item `id` is stored at slot id, laid out [d][column]
    const size_t slot = static_cast<size_t>(id);
    if constexpr (MODE == 2) {
        // column waves hold their tile's whole partial: store it as it is
        lcw = colsum4(lcw);
        const int colw = w * 16 + col16;
        if (w < NCT && colw < ncols) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int ee = 0; ee < 4; ++ee)
                    st_coh(p.part_o + (slot * D + dt * 16 + kg * 4 + ee) * p.CPG + colw, ocw[dt][ee]);
            if (kg == 0) {
                const unsigned long long v =
                    (static_cast<unsigned long long>(__float_as_uint(lcw)) << 32) | __float_as_uint(mcw);
                st_coh(reinterpret_cast<unsigned long long*>(p.part_ml + slot * p.CPG + colw), v);
            }
        }
    }
    if constexpr (MODE != 2) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            __syncthreads();
            if (kg == 0 && half == 0) {
                S.red.m[w][col16] = mrun[ct];
                S.red.l[w][col16] = lrun[ct];
            }
#pragma unroll
            for (int dt = half * (DT / 2); dt < (half + 1) * (DT / 2); ++dt)
#pragma unroll
                for (int ee = 0; ee < 4; ++ee)
                    S.red.o[w][(dt - half * (DT / 2)) * 16 + kg * 4 + ee][col16] = o[ct][dt][ee];
            __syncthreads();
            const int ncol = min(16, ncols - ct * 16);
            for (int idx = tid; idx < 16 * (D / 2); idx += kThreads) {
                const int cl = idx & 15, dh = idx >> 4;
                if (cl >= ncol) continue;
                const int col = ct * 16 + cl, d = half * (D / 2) + dh;
                float ms = -INFINITY;
#pragma unroll
                for (int u = 0; u < 4; ++u) ms = fmaxf(ms, S.red.m[u][cl]);
                float accv = 0.0f, l = 0.0f;
                if (ms != -INFINITY) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float mu = S.red.m[u][cl];
                        const float f = (mu == -INFINITY) ? 0.0f : exp2f(mu - ms);
                        accv += S.red.o[u][dh][cl] * f;
                        l += S.red.l[u][cl] * f;
                    }
                }
                st_coh(p.part_o + (slot * D + d) * p.CPG + col, accv);
                if (d == 0) {
                    const unsigned long long v =
                        (static_cast<unsigned long long>(__float_as_uint(l)) << 32) | __float_as_uint(ms);
                    st_coh(reinterpret_cast<unsigned long long*>(p.part_ml + slot * p.CPG + col), v);
                }
            }
        }
    }
    }
    if (arrive_last(p.merge_cnt + static_cast<size_t>(b) * p.Hkv + g, qb, &S.flag))
        dec_merge<D, NCT>(p, S.mrg, b, g, first_slot + g, p.Hkv, qb, q0, k1);
}

// ---- Column waves over an even split of the keys (grouped heads, D = 128).
//
// The 32-key items of all sequences are laid end to end (N in all, one kv
// head's worth) and cut into W equal ranges; workgroup r * Hkv + g takes range
// r of kv head g, so every resident workgroup gets the same work in one round
// and the Hkv workgroups of a range, dispatched together, read the same cache
// rows at the same time.  (Per-sequence chunks of at most 192 16-key slices
// need about 1.6 rounds on the B=64, K=8 workload, and each workgroup streams
// at the same rate whether the round is full or not, so the partly filled
// second round took as long as a full one.)  A range meets one or more
// sequences; its part of sequence b is a piece with its own partial at slot
// (r + b) * Hkv + g, so the pieces of a (sequence, kv head) sit Hkv slots
// apart and no two pieces share a slot.  The pieces pass through a four-slot
// ring (three items in flight, 16 KB each) as one stream of items: for each
// piece its query item (all its column tiles), then its key items.  Each
// compute wave takes a whole 32-key item per step: two independent 16-key
// score chains, one online softmax step and 32-key PV products, which halves
// the dependent steps and barriers per key of a 16-key step.  Each wave counts
// the vector memory operations it issues (ring loads and partial stores; they
// complete in issue order), so the wait for an item is exact even when a
// piece's partial stores sit between it and the later items.  A piece that is
// all of its sequence (no shared prefix) writes the output itself; for the
// others, at its end the workgroup counts itself in the arrival counter of
// their (sequence, kv head) pairs, and the last arriver merges that pair's
// pieces.
constexpr int kPieceMax = 8;
constexpr int kStreamMerge = 512;  // (part, column) pairs a merge stages in LDS at a time
constexpr int kStreamSlots = 4;    // ring slots: three 32-key items in flight

// One ring slot of the even-split kernel: 32 K rows and the same 32 V rows
// (16-byte chunk c of row r at c ^ prefix_swz(r)), or 64 query rows.
struct StreamSlot {
    uint4 k[32 * 16];
    uint4 v[32 * 16];
};

struct StreamPiece {
    int b, g;      // sequence, kv head
    int lo, n;     // first 32-key item of the piece; its items with keys on the device (-1: bad sequence)
    int L, q0, k1; // device cache length, first query row, query rows
    int whole;     // the piece is all of the sequence and there is no shared prefix:
                   // its result is the output
    long long kv0; // first cache row of the sequence
};

struct DecLdsStream {
    struct {
        float2 ml[kStreamMerge];
        float w[kStreamMerge];
    } mrg;
    StreamPiece pc[kPieceMax];
    int np;
    int last[kPieceMax];
};

// A position in a workgroup's item stream: piece k, item i of its `items`
// (the query item, then the piece's key items), and the piece's parameters as
// wave-uniform values.
struct StreamCursor {
    int k, i, items;
    int b, g, lo, n, L, q0, k1, whole;
    long long kv0;
};

__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform_i64(long long v) {
    return static_cast<long long>(
        (static_cast<unsigned long long>(static_cast<unsigned>(uniform_i32(static_cast<int>(v >> 32))))
         << 32) |
        static_cast<unsigned>(uniform_i32(static_cast<int>(v))));
}

// Piece k's parameters into the cursor (item 0).
__device__ __forceinline__ void stream_at(StreamCursor& c, const DecLdsStream& S, int k) {
    const StreamPiece& P = S.pc[k];
    c.k = k;
    c.i = 0;
    c.b = uniform_i32(P.b);
    c.g = uniform_i32(P.g);
    c.lo = uniform_i32(P.lo);
    c.n = uniform_i32(P.n);
    c.L = uniform_i32(P.L);
    c.q0 = uniform_i32(P.q0);
    c.k1 = uniform_i32(P.k1);
    c.whole = uniform_i32(P.whole);
    c.kv0 = uniform_i64(P.kv0);
    c.items = c.n > 0 ? 1 + c.n : 0;
}

// This wave's four 16-byte loads of an item: rows r0 = 8w + lane/16 and
// r1 = r0 + 4 of both halves of a slot, from 16-byte chunks c0, c1 of their
// source rows (the row swizzle applied on the load side); off0, off1: their
// element offsets from an item's first cache row.
struct StreamLoadLanes {
    int dst, r0, r1, c0, c1, off0, off1;
};

// Issue this wave's loads of the cursor's current item into slot R: the
// query item (columns 0-31 in the K half, 32-63 in the V half; padding
// columns repeat the last column, finite and never stored), or 32 keys.
__device__ __forceinline__ void stream_issue(const AttnParams& p, StreamSlot& R, const StreamCursor& c,
                                             const StreamLoadLanes& ln) {
    constexpr int D = 128;
    const uint16_t *k0p, *k1p, *v0p, *v1p;
    if (c.i == 0) {
        const int ncl = p.G * c.k1;
        int col[4] = {ln.r0, ln.r1, 32 + ln.r0, 32 + ln.r1};
        const uint16_t* src[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int cl = min(col[u], ncl - 1);
            src[u] = p.q + (static_cast<size_t>(c.q0 + cl % c.k1) * p.Hq + c.g * p.G + cl / c.k1) * D +
                     ((u & 1) ? ln.c1 : ln.c0) * 8;
        }
        k0p = src[0];
        k1p = src[1];
        v0p = src[2];
        v1p = src[3];
    } else if ((c.lo + c.i - 1) * 32 + 31 < c.L) {
        // every row of the item is a cache row: a uniform base
        const size_t base = static_cast<size_t>(c.kv0 + (c.lo + c.i - 1) * 32) * p.Hkv * D;
        k0p = p.k_cache + base + ln.off0;
        k1p = p.k_cache + base + ln.off1;
        v0p = p.v_cache + base + ln.off0;
        v1p = p.v_cache + base + ln.off1;
    } else {
        // keys < L are cache rows, the next k1 the new rows; keys past the
        // last one are clamped to it (and masked)
        const int k0 = (c.lo + c.i - 1) * 32;
        const int T = c.L + c.k1;
        const int t0 = min(k0 + ln.r0, T - 1), t1 = min(k0 + ln.r1, T - 1);
        const size_t rs = static_cast<size_t>(p.Hkv) * D, head = static_cast<size_t>(c.g) * D;
        const size_t o0 = ((t0 < c.L) ? static_cast<size_t>(c.kv0 + t0) : 0) * rs + head + ln.c0 * 8;
        const size_t n0 = static_cast<size_t>(c.q0 + (t0 - c.L)) * rs + head + ln.c0 * 8;
        const size_t o1 = ((t1 < c.L) ? static_cast<size_t>(c.kv0 + t1) : 0) * rs + head + ln.c1 * 8;
        const size_t n1 = static_cast<size_t>(c.q0 + (t1 - c.L)) * rs + head + ln.c1 * 8;
        k0p = (t0 < c.L) ? p.k_cache + o0 : p.k_new + n0;
        v0p = (t0 < c.L) ? p.v_cache + o0 : p.v_new + n0;
        k1p = (t1 < c.L) ? p.k_cache + o1 : p.k_new + n1;
        v1p = (t1 < c.L) ? p.v_cache + o1 : p.v_new + n1;
    }
    __builtin_amdgcn_global_load_lds(k0p, R.k + ln.dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(k1p, R.k + ln.dst + 64, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(v0p, R.v + ln.dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(v1p, R.v + ln.dst + 64, 16, 0, 0);
}

// Running state of a column wave's tile over the current piece.
template <int KK, int DT>
struct StreamTile {
    float m, l;
    floatx4 o[DT];
    bf16x8 qv[KK];
};

// Store the compute wave's tile partial at `slot` -- or, for a piece that is
// all of its sequence (`whole`), the normalised output rows q0 + j of heads
// g*G + hh -- and reset the state.  Returns the vector memory operations
// issued, counted low: the (m, l) store, issued only where kg == 0, is left
// out.
template <int KK, int DT>
__device__ __forceinline__ int stream_store(const AttnParams& p, StreamTile<KK, DT>& t, bool cw, int w,
                                            int colw, int kg, size_t slot, int ncl, bool whole, int q0,
                                            int k1, int g) {
    constexpr int D = 128;
    int ops = 0;
    t.l = colsum4(t.l);
    // (opaque copies of the lane's column and key group: the store addresses
    // are formed here, not hoisted out of the item loop where they would hold
    // registers)
    asm volatile("" : "+v"(colw), "+v"(kg));
    if (whole) {
        // a single part: the merge would weight it by exactly 1 / l
        if (cw && w * 16 < ncl) {
            if (colw < ncl) {
                const float inv = 1.0f / t.l;
                const int hh = colw / k1, j = colw - hh * k1;
                uint16_t* orow = static_cast<uint16_t*>(p.out) +
                                 (static_cast<size_t>(q0 + j) * p.Hq + g * p.G + hh) * D + kg * 4;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const unsigned lo = f32_to_bf16(t.o[dt][0] * inv) | (f32_to_bf16(t.o[dt][1] * inv) << 16);
                    const unsigned hi = f32_to_bf16(t.o[dt][2] * inv) | (f32_to_bf16(t.o[dt][3] * inv) << 16);
                    *reinterpret_cast<uint2*>(orow + dt * 16) = make_uint2(lo, hi);
                }
            }
            ops = DT;
        }
    } else if (cw && w * 16 < ncl) {
        if (colw < ncl) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int ee = 0; ee < 4; ++ee)
                    st_coh(p.part_o + (slot * D + dt * 16 + kg * 4 + ee) * p.CPG + colw, t.o[dt][ee]);
            if (kg == 0) {
                const unsigned long long v =
                    (static_cast<unsigned long long>(__float_as_uint(t.l)) << 32) | __float_as_uint(t.m);
                st_coh(reinterpret_cast<unsigned long long*>(p.part_ml + slot * p.CPG + colw), v);
            }
        }
        ops = DT * 4;
    }
    t.m = -INFINITY;
    t.l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) t.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    return ops;
}

// s_waitcnt vmcnt(n) for a wave-uniform n computed at run time (n > 63: 63).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define SV_VMC(c) case c: __builtin_amdgcn_s_waitcnt(0x0F70 | ((c) & 15) | (((c) >> 4) << 14)); break;
#define SV_VMC8(c) SV_VMC(c) SV_VMC(c + 1) SV_VMC(c + 2) SV_VMC(c + 3) SV_VMC(c + 4) SV_VMC(c + 5) \
    SV_VMC(c + 6) SV_VMC(c + 7)
    switch (n) {
        SV_VMC8(0) SV_VMC8(8) SV_VMC8(16) SV_VMC8(24) SV_VMC8(32) SV_VMC8(40) SV_VMC8(48)
        SV_VMC(56) SV_VMC(57) SV_VMC(58) SV_VMC(59) SV_VMC(60) SV_VMC(61) SV_VMC(62)
        default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15 | (3 << 14)); break;
    }
#undef SV_VMC8
#undef SV_VMC
}

// The range that holds slice x of the even split.
__device__ __forceinline__ int stream_owner(long long x, int W, long long N) {
    return static_cast<int>(((x + 1) * W - 1) / N);
}

template <int NCT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_stream_kernel(AttnParams p, DecPlan plan) {
    constexpr int D = 128;
    constexpr int KK = D / 32, DT = D / 16;
    __shared__ DecLdsStream S;
    __shared__ StreamSlot C0, C1, C2, C3;  // kStreamSlots slots

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col16 = lane & 15, kg = lane >> 4;
    const int Hkv = p.Hkv, W = plan.W;
    const int wg = blockIdx.x, rg = wg / Hkv, hg = wg - rg * Hkv;  // range, kv head
    const long long N = plan.N;
    const long long x0 = static_cast<long long>(rg) * N / W;
    const long long x1 = static_cast<long long>(rg + 1) * N / W;

    // ---- the pieces of [x0, x1): wave 0, lane k records piece k
    if (w == 0) {
        int pb = 0, plo = 0, phi = 0, np = 0;
        long long x = x0;
        while (x < x1 && np < kPieceMax) {
            int cnt = 0;  // sequence of item x: the sequences whose items all precede it
            for (int b0 = 0; b0 < plan.nb; b0 += 64) {
                const int bb = b0 + lane;
                cnt += __popcll(__ballot((bb < plan.nb) && plan.q[bb + 1] <= x));
            }
            const int b = uniform_i32(cnt);
            const int lo = static_cast<int>(x - plan.q[b]);
            const int len = static_cast<int>(min(static_cast<long long>(plan.s[b] - lo), x1 - x));
            if (lane == np) {
                pb = b;
                plo = lo;
                phi = lo + len;
            }
            ++np;
            x += len;
        }
        if (x < x1 && lane == 0) set_status(p.status, 3);  // more pieces than the host plan allows
        if (lane < np) {
            // the sequence's device data: every workgroup of a sequence takes
            // the same decision, so a bad sequence arrives nowhere
            const int q0 = plan.row0[pb], k1 = plan.row0[pb + 1] - q0;
            const int L = p.kv_len[pb];
            const long long kv0 = p.kv_start[pb];
            bool bad = (L < 0) || (static_cast<long long>(L) + k1 > 32LL * plan.s[pb]);
            if (p.cu_q) bad = bad || (p.cu_q[pb] != q0) || (p.cu_q[pb + 1] != q0 + k1);
            if (bad) set_status(p.status, 3);
            const int n = bad ? -1 : max(0, min(phi, ceil_div(L + k1, 32)) - plo);
            // (with a shared prefix every piece is merged with the prefix parts)
            const int whole = (p.prefix_slots == 0 && plo == 0 && phi == plan.s[pb]) ? 1 : 0;
            S.pc[lane] = StreamPiece{pb, hg, plo, n, L, q0, k1, whole, kv0};
        }
        if (lane == 0) S.np = np;
    }
    __syncthreads();
    const int np = S.np;
    int nitems = 0;
    for (int k = 0; k < np; ++k) {
        const int n = S.pc[k].n;
        nitems += n > 0 ? 1 + n : 0;
    }

    // loads: wave w fills rows 8w .. 8w+7 of both halves of a slot
    StreamLoadLanes ln;
    ln.dst = 2 * w * 64;
    ln.r0 = 8 * w + (lane >> 4);
    ln.r1 = ln.r0 + 4;
    ln.c0 = (lane & 15) ^ prefix_swz(ln.r0);
    ln.c1 = (lane & 15) ^ prefix_swz(ln.r1);
    ln.off0 = ln.r0 * Hkv * D + hg * D + ln.c0 * 8;
    ln.off1 = ln.r1 * Hkv * D + hg * D + ln.c1 * 8;
    // the loader's cursor: at the first piece with items
    StreamCursor lc{};
    lc.k = -1;
    for (int k = 0; k < np && lc.k < 0; ++k)
        if (S.pc[k].n > 0) stream_at(lc, S, k);
    auto lnext = [&]() __attribute__((always_inline)) {
        if (++lc.i == lc.items) {
            int k = lc.k + 1;
            while (k < np && S.pc[k].n <= 0) ++k;
            if (k < np) stream_at(lc, S, k);
        }
    };

    // compute: wave w < NCT holds column tile w of the current piece
    const bool cw = w < NCT;
    const int colw = w * 16 + col16;
    // K operand of a slot: row col16, logical chunk kg + 4 kk, at (kg ^ (sk &
    // 3)) + 4 (kk ^ (sk >> 2)); V^T operand: row kg*4 + col16/4 (as the
    // grouped-head ring of decode_bf16_kernel)
    const int csk = prefix_swz(col16);
    const int ckcol = col16 * 16 + (kg ^ (csk & 3));
    const int csk2 = csk >> 2;
    const int crv = kg * 4 + (col16 >> 2);
    const int csv = prefix_swz(crv);
    const int csv1 = csv >> 1;
    const int cvcol = crv * D + 8 * (((col16 & 3) >> 1) ^ (csv & 1)) + 4 * (col16 & 1);
    StreamTile<KK, DT> t;
    t.m = -INFINITY;
    t.l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) t.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) t.qv[kk] = bf16x8{};
    int iss = 0;  // vector memory operations this wave has issued (counted low)
    // the compute cursor: pieces of no slice on the device before the first
    // piece with items store an empty partial (their segment counts them),
    // bad sequences nothing
    StreamCursor cc{};
    cc.k = -1;
    int climw = 0;  // causal limit of this lane's column in the current piece
    for (int k = 0; k < np && cc.k < 0; ++k) {
        const int n = S.pc[k].n;
        if (n > 0) {
            stream_at(cc, S, k);
            climw = (cw && colw < p.G * cc.k1) ? cc.L + colw % cc.k1 + 1 : 0;
        } else if (n == 0) {
            iss += stream_store<KK, DT>(p, t, cw, w, colw, kg, static_cast<size_t>(rg + S.pc[k].b) * Hkv + hg,
                                        p.G * S.pc[k].k1, false, 0, 1, hg);
        }
    }
    // The first piece that ends before the stream does and is not a whole
    // sequence is counted in its arrival counter early, once the loads of a
    // later item have been waited for (its partial stores, issued before
    // them, are then complete in every wave): the workgroup of the range
    // before this one, whose last piece shares the pair and ends later, is
    // then the one that merges it, and no workgroup merges two pairs at its
    // end.  (0: none yet, 1: stores issued, 2: counted; `early_old` holds the
    // count before it in lane early_k of wave 0.)
    int early_state = 0, early_k = 0, early_iss = 0, early_old = 0;
    auto cnext = [&]() __attribute__((always_inline)) {
        if (++cc.i == cc.items) {
            // the piece is done: its partial, then those of the empty pieces
            // up to the next one with items
            iss += stream_store<KK, DT>(p, t, cw, w, colw, kg, static_cast<size_t>(rg + cc.b) * Hkv + hg,
                                        p.G * cc.k1, cc.whole != 0, cc.q0, cc.k1, hg);
            if (early_state == 0 && cc.whole == 0) {
                early_state = 1;
                early_k = cc.k;
                early_iss = iss;
            }
            int k = cc.k + 1;
            for (; k < np && S.pc[k].n <= 0; ++k)
                if (S.pc[k].n == 0)
                    iss += stream_store<KK, DT>(p, t, cw, w, colw, kg,
                                                static_cast<size_t>(rg + S.pc[k].b) * Hkv + hg,
                                                p.G * S.pc[k].k1, false, 0, 1, hg);
            if (k < np) {
                stream_at(cc, S, k);
                climw = (cw && colw < p.G * cc.k1) ? cc.L + colw % cc.k1 + 1 : 0;
            }
        }
    };
    // item in slot R: the query tiles into registers, or 32 keys' products:
    // S^T of the two 16-key halves (two independent chains), one online
    // softmax step over all 32, and O^T += V^T P^T with 32 keys per product,
    // lane group kg supplying keys kg*4 + 0..3 of the first half, then of the
    // second, on both operands (the same order, so every key is summed once)
    auto compute = [&](StreamSlot& R) __attribute__((always_inline)) {
        if (cc.i == 0) {
            if (cw) {
                const uint4* src = (w < 2 ? R.k : R.v) + (w & 1) * 256;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    t.qv[kk] = *reinterpret_cast<const bf16x8*>(src + ckcol + 4 * (kk ^ csk2));
            }
        } else if (cw) {
            const int k0 = (cc.lo + cc.i - 1) * 32;
            floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                bf16x8 ka[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    ka[h] = *reinterpret_cast<const bf16x8*>(R.k + h * 256 + ckcol + 4 * (kk ^ csk2));
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[h], t.qv[kk], acc[h], 0, 0, 0);
            }
            const bool full = k0 + 31 < cc.L;  // no key of the item is masked for any column
            float mt = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tt = k0 + h * 16 + kg * 4 + e;
                    acc[h][e] = (full || tt < climw) ? acc[h][e] * p.scale_log2 : -INFINITY;
                    mt = fmaxf(mt, acc[h][e]);
                }
            mt = colmax4(mt);
            const float mnew = fmaxf(t.m, mt);
            // no column of the tile raised its running max: alpha is exactly 1
            // on every lane and the rescale of O is skipped
            const bool grew = __ballot(mt > t.m) != 0;
            shortx4 pb[2] = {shortx4{0, 0, 0, 0}, shortx4{0, 0, 0, 0}};
            float alpha = 1.0f;
            if (mnew != -INFINITY) {  // (a padding column has no key)
                if (grew) alpha = __builtin_amdgcn_exp2f(t.m - mnew);
                float ps = 0.0f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pe = __builtin_amdgcn_exp2f(acc[h][e] - mnew);
                        ps += pe;
                        pb[h][e] = static_cast<short>(f32_to_bf16(pe));
                    }
                t.l = t.l * alpha + ps;
                t.m = mnew;
            }
            if (grew) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) t.o[dt] *= alpha;
            }
            const bf16x8 pk = __builtin_bit_cast(
                bf16x8, (shortx8{pb[0][0], pb[0][1], pb[0][2], pb[0][3], pb[1][0], pb[1][1], pb[1][2], pb[1][3]}));
            const uint16_t* vb = reinterpret_cast<const uint16_t*>(R.v);
#pragma unroll
            for (int d0 = 0; d0 < DT; d0 += 4) {
                bf16x8 va[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const shortx4 a0 = lds_read_tr16(vb + cvcol + 16 * ((d0 + u) ^ csv1));
                    const shortx4 a1 = lds_read_tr16(vb + 16 * D + cvcol + 16 * ((d0 + u) ^ csv1));
                    va[u] = __builtin_bit_cast(bf16x8, (shortx8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    t.o[d0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], pk, t.o[d0 + u], 0, 0, 0);
            }
        }
    };

    constexpr int AHEAD = kStreamSlots - 1;  // items in flight
    constexpr int kOps = 4;                  // loads per wave per item
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;      // iss after each slot's loads
#define SV_ISSUE(R, A)                     \
    do {                                   \
        stream_issue(p, R, lc, ln);        \
        lnext();                           \
        iss += kOps;                       \
        A = iss;                           \
    } while (0)
    // one ring step: item j is in once this wave's loads of it are done and
    // every wave passed the barrier; slot Rn (item j-1) is then free for
    // item j + AHEAD
#define SV_STEP(J, R, Rn, A, An)                                      \
    do {                                                              \
        {                                                             \
            const int vm_ = uniform_i32(iss - (A));                   \
            if (vm_ == kOps * (AHEAD - 1)) __builtin_amdgcn_s_waitcnt(0x0F70 | (kOps * (AHEAD - 1))); \
            else wait_vmcnt(vm_);                                     \
        }                                                             \
        __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): LDS reads done */ \
        __builtin_amdgcn_s_barrier();                                 \
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); \
        if (early_state == 1 && (A) > early_iss) {                    \
            early_state = 2;                                          \
            if (tid == early_k)                                       \
                early_old = __hip_atomic_fetch_add(                   \
                    p.merge_cnt + static_cast<size_t>(S.pc[early_k].b) * Hkv + S.pc[early_k].g, 1, \
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);      \
        }                                                             \
        if ((J) + AHEAD < nitems) SV_ISSUE(Rn, An);                   \
        compute(R);                                                   \
        cnext();                                                      \
    } while (0)
    static_assert(kStreamSlots == 4 && kOps * (AHEAD - 1) < 16, "the ring below has four slots");
    if (nitems > 0) SV_ISSUE(C0, a0);
    if (nitems > 1) SV_ISSUE(C1, a1);
    if (nitems > 2) SV_ISSUE(C2, a2);
    for (int j = 0; j < nitems; j += 4) {
        SV_STEP(j, C0, C3, a0, a3);
        if (j + 1 < nitems) SV_STEP(j + 1, C1, C0, a1, a0);
        if (j + 2 < nitems) SV_STEP(j + 2, C2, C1, a2, a1);
        if (j + 3 < nitems) SV_STEP(j + 3, C3, C2, a3, a2);
    }
#undef SV_STEP
#undef SV_ISSUE

    // ---- arrivals: every partial of this workgroup is stored; count it in
    // the (sequence, kv head) of each piece that is not the whole sequence
    // (nor of a bad one); the last arriver merges that pair's pieces
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid < np) {  // lane k of wave 0: piece k (the counts in one round trip)
        const StreamPiece& P = S.pc[tid];
        int last = 0;
        if (P.n >= 0 && !P.whole) {
            const long long st = plan.q[P.b];
            const int parts = stream_owner(st + plan.s[P.b] - 1, W, N) - stream_owner(st, W, N) + 1;
            int* cnt = p.merge_cnt + static_cast<size_t>(P.b) * Hkv + P.g;
            const int old = (early_state == 2 && tid == early_k)
                                ? early_old
                                : __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (old == parts - 1) ? 1 : 0;
            if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        S.last[tid] = last;
    }
    __syncthreads();
    for (int k = 0; k < np; ++k) {
        if (!S.last[k]) continue;
        const int b = S.pc[k].b;
        const long long st = plan.q[b];
        const int r_lo = stream_owner(st, W, N);
        const int parts = stream_owner(st + plan.s[b] - 1, W, N) - r_lo + 1;
        dec_merge<D, NCT>(p, S.mrg, b, hg, (r_lo + b) * Hkv + hg, Hkv, parts, S.pc[k].q0, S.pc[k].k1);
    }
}

template <int D>
struct PrefixLds {
    static constexpr int KP = D + 8;  // K tile pitch (bf16)
    static constexpr int VP = D + 4;  // V tile pitch (bf16)
    static constexpr int kTile = 128; // keys per tile (two halves of 64 for the products)
    alignas(16) uint16_t ks[kTile][KP];  // rows of KP*2 = 16*(D/8+1) bytes: 16-byte reads
    uint16_t vs[kTile][VP];
};

// grid: x = prefix chunk, y = kv head, z = column group (16 tiles of 16 columns);
// block: 16 waves, one per column tile of the group (waves past the group's
// tiles only help load the K/V tiles).
template <int D>
__global__ __launch_bounds__(1024) void prefix_bf16_kernel(AttnParams p) {
    constexpr int KK = D / 32, DT = D / 16, VCH = D / 8;
    __shared__ PrefixLds<D> S;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nthreads = blockDim.x;
    const int x = blockIdx.x, g = blockIdx.y;
    const int t_begin = x * p.prefix_chunk;
    const int t_end = min(p.prefix_len, t_begin + p.prefix_chunk);
    const int col16 = lane & 15, kg = lane >> 4;
    const int tile = blockIdx.z * 16 + w;
    const int cg = tile * 16 + col16;           // global column: b*CPG + hh*(K_b+1) + j
    const bool active = tile * 16 < p.NC;
    int k1c = 1, q0c = 0;                       // the column's sequence
    if (cg < p.NC) {
        k1c = seq_k1(p, cg / p.CPG);
        q0c = seq_q0(p, cg / p.CPG);
    }
    const bool col_ok = (cg < p.NC) && (cg % p.CPG < p.G * k1c);

    bf16x8 qv[KK];
    if (col_ok) {
        const int cl = cg % p.CPG;
        const int hh = cl / k1c, j = cl % k1c;
        const uint16_t* qp =
            p.q + (static_cast<size_t>(q0c + j) * p.Hq + g * p.G + hh) * D + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[kk][e] = static_cast<__bf16>(0.0f);
    }

    floatx4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f;
    const size_t row_stride = static_cast<size_t>(p.Hkv) * D;

    // One K and V tile of kTile keys is 2*kTile*VCH 16-byte words.  With at
    // least 2*kTile*VCH/kPL threads every thread holds its words of the next
    // tile in registers: they are issued before the current tile's products
    // and written to LDS after them, so the loads overlap the MFMA work.
    constexpr int kTile = PrefixLds<D>::kTile;
    constexpr int kPL = 4;
    constexpr int kWords = 2 * kTile * VCH;
    const bool staged = kWords <= kPL * nthreads;
    auto word_src = [&](int qi, int tb) -> const uint4* {
        const int isv = qi >= kTile * VCH;
        const int r = (qi % (kTile * VCH)) / VCH, dc = qi % VCH;
        const int t = min(tb + r, p.prefix_len - 1);
        return reinterpret_cast<const uint4*>((isv ? p.v_prefix : p.k_prefix) +
                                              static_cast<size_t>(t) * row_stride +
                                              static_cast<size_t>(g) * D + dc * 8);
    };
    auto word_put = [&](int qi, uint4 v) {
        const int isv = qi >= kTile * VCH;
        const int r = (qi % (kTile * VCH)) / VCH, dc = qi % VCH;
        if (isv) {
            uint2* dst = reinterpret_cast<uint2*>(&S.vs[r][dc * 8]);  // V rows are 8-byte aligned
            dst[0] = make_uint2(v.x, v.y);
            dst[1] = make_uint2(v.z, v.w);
        } else {
            *reinterpret_cast<uint4*>(&S.ks[r][dc * 8]) = v;
        }
    };
    uint4 nx[kPL];
    auto issue = [&](int tb) {
#pragma unroll
        for (int u = 0; u < kPL; ++u) {
            const int qi = tid + u * nthreads;
            if (qi < kWords) nx[u] = *word_src(qi, tb);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int u = 0; u < kPL; ++u) {
            const int qi = tid + u * nthreads;
            if (qi < kWords) word_put(qi, nx[u]);
        }
    };
    // transposed-read address of this lane in a 16-key sub-tile of V (as in
    // the decode kernel): row kg*4 + col16/4, column 4*(col16%4)
    const uint16_t* vt_lane = &S.vs[kg * 4 + (col16 >> 2)][(col16 & 3) * 4];

    if (staged && t_begin < t_end) {
        issue(t_begin);
        stash();
    }
    for (int tb = t_begin; tb < t_end; tb += kTile) {
        if (!staged) {
            // cooperative load of the K and V tiles
            for (int qi = tid; qi < kWords; qi += nthreads) word_put(qi, *word_src(qi, tb));
        }
        __syncthreads();
        const bool more = staged && (tb + kTile < t_end);
        if (more) issue(tb + kTile);  // in flight during this tile's products
#pragma unroll 1
        for (int half = 0; half < kTile / 64; ++half) {
        const int hb = tb + half * 64;   // first key of the half
        if (active && hb < t_end) {
            floatx4 acc[4];
            float mt = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) acc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
            // one slice of D at a time: two 16-key operands are read together,
            // then feed two independent products
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int k0 = 0; k0 < 4; k0 += 2) {
                    bf16x8 ka[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        ka[u] = *reinterpret_cast<const bf16x8*>(
                            &S.ks[half * 64 + (k0 + u) * 16 + col16][kg * 8 + 32 * kk]);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acc[k0 + u] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qv[kk], acc[k0 + u], 0, 0, 0);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = hb + kt * 16 + kg * 4 + e;
                    acc[kt][e] = (t < t_end) ? acc[kt][e] * p.scale_log2 : -INFINITY;
                    mt = fmaxf(mt, acc[kt][e]);
                }
            }
            mt = colmax4(mt);
            const float mnew = fmaxf(mrun, mt);   // finite: every half computed has a valid key
            // no column of the tile raised its running max: alpha is exactly 1
            // on every lane and the rescale of O is skipped
            const bool grew = __ballot(mt > mrun) != 0;
            const float alpha = grew ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
            float ps = 0.0f;
            shortx4 pb[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(acc[kt][e] - mnew);
                    ps += pe;
                    pb[kt][e] = static_cast<short>(f32_to_bf16(pe));
                }
            lrun = lrun * alpha + ps;
            mrun = mnew;
            if (grew) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                // V^T operands of 16 keys: lane (d = dt*16 + col16) gets keys
                // kt*16 + kg*4 .. +3; four reads issue before their products
#pragma unroll
                for (int d0 = 0; d0 < DT; d0 += 4) {
                    shortx4 va[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        va[u] = lds_read_tr16(vt_lane + (half * 64 + kt * 16) * PrefixLds<D>::VP +
                                              (d0 + u) * 16);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        o[d0 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[u], pb[kt], o[d0 + u], 0, 0, 0);
                }
            }
        }
        }  // half
        __syncthreads();  // every wave is done with the tile
        if (more) stash();
    }
    lrun = colsum4(lrun);
    if (cg < p.NC) {
        const size_t base = (static_cast<size_t>(x) * p.Hkv + g) * p.NC + cg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.pre_o[base * D + dt * 16 + kg * 4 + e] = o[dt][e];
        if (kg == 0) p.pre_ml[base] = make_float2(mrun, lrun);
    }
}

// D = 128 form of the prefix kernel whose K/V tiles reach LDS through the
// direct global-to-LDS load (global_load_lds_dwordx4): two tile buffers, one
// barrier per tile and no staging registers.  Each wave-wide load writes
// 64 x 16 contiguous bytes of LDS, so rows are stored unpadded (256 bytes);
// the 16-byte chunk c of row r is stored at position c ^ swz(r), which puts
// the 16-byte K reads of 16 consecutive rows and the transposed 8-byte V reads
// of 16 rows x 2 chunks on distinct LDS banks.
// One tile buffer; the kernel holds two as separate LDS objects, so the
// compiler can tell reads of one from direct loads still landing in the other.
struct PrefixDmaBuf {
    static constexpr int kTile = 128;   // keys per tile
    static constexpr int kChunks = 16;  // 16-byte chunks per 128-wide bf16 row
    uint4 k[kTile * kChunks];
    uint4 v[kTile * kChunks];
};


// grid as for prefix_bf16_kernel; block: 1024 threads (16 waves), which the
// mapping of waves to column tiles below assumes.
__global__ __launch_bounds__(1024) void prefix_dma_kernel(AttnParams p) {
    constexpr int D = 128, KK = D / 32, DT = D / 16;
    constexpr int kTile = PrefixDmaBuf::kTile, kCh = PrefixDmaBuf::kChunks;
    constexpr int kBlocks = 2 * kTile * kCh / 64;  // 1 KB blocks of K and V per tile
    __shared__ PrefixDmaBuf SA, SB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int x = blockIdx.x, g = blockIdx.y;
    const int t_begin = x * p.prefix_chunk;
    const int t_end = min(p.prefix_len, t_begin + p.prefix_chunk);
    const int col16 = lane & 15, kg = lane >> 4;
    // Waves to column tiles: with more than 8 tiles in the group, 16 - ntiles
    // of them are split so that two waves take one 64-key half of every K/V
    // tile each (10 tiles: 4 whole + 12 half waves, five half-tile units on
    // each SIMD instead of 3/3/2/2 whole tiles); with at most 8, all are
    // split.  A split pair merges its two softmax states at the end.
    const int ntiles = min(16, (p.NC + 15) / 16 - static_cast<int>(blockIdx.z) * 16);
    const int nsplit = ntiles <= 8 ? ntiles : 16 - ntiles;
    const int nwhole = ntiles - nsplit;
    const int tile_l = w < nwhole ? w : nwhole + (w - nwhole) / 2;
    const int myhalf = w < nwhole ? -1 : (w - nwhole) & 1;  // -1: both halves
    const int tile = blockIdx.z * 16 + tile_l;
    const int cg = tile * 16 + col16;           // global column: b*CPG + hh*(K_b+1) + j
    const bool active = tile_l < ntiles;
    int k1c = 1, q0c = 0;                       // the column's sequence
    if (active && cg < p.NC) {
        k1c = seq_k1(p, cg / p.CPG);
        q0c = seq_q0(p, cg / p.CPG);
    }
    const bool col_ok = active && (cg < p.NC) && (cg % p.CPG < p.G * k1c);

    bf16x8 qv[KK];
    if (col_ok) {
        const int cl = cg % p.CPG;
        const int hh = cl / k1c, j = cl % k1c;
        const uint16_t* qp =
            p.q + (static_cast<size_t>(q0c + j) * p.Hq + g * p.G + hh) * D + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[kk][e] = static_cast<__bf16>(0.0f);
    }

    floatx4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f;
    const size_t row_stride = static_cast<size_t>(p.Hkv) * D;

    // block b of a tile: K rows 4b..4b+3 (b < kBlocks/2), else V rows of
    // b - kBlocks/2; lane l fills row 4*(b mod kBlocks/2) + l/16, position l%16
    const int lrow = lane >> 4, lpos = lane & 15;
    auto issue = [&](int tb, PrefixDmaBuf& B) {
        for (int b = w; b < kBlocks; b += nwaves) {
            const int isv = b >= kBlocks / 2;
            const int bb = isv ? b - kBlocks / 2 : b;
            const int r = bb * 4 + lrow;
            const int c = lpos ^ prefix_swz(r);
            const int t = min(tb + r, p.prefix_len - 1);
            const uint16_t* src = (isv ? p.v_prefix : p.k_prefix) + static_cast<size_t>(t) * row_stride +
                                  static_cast<size_t>(g) * D + c * 8;
            uint4* dst = (isv ? B.v : B.k) + bb * 64;
            __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
        }
    };
    // K operand: row half*64 + kt*16 + col16 (row mod 16 = col16), logical
    // chunk kg + 4*kk, stored at (kg ^ (sk & 3)) + 4*(kk ^ (sk >> 2))
    const int sk = prefix_swz(col16);
    const int kcol = col16 * kCh + (kg ^ (sk & 3));
    const int sk2 = sk >> 2;
    // V^T operand: row half*64 + kt*16 + rv with rv = kg*4 + col16/4, logical
    // chunk 2*dt + h (h = (col16 & 3) >> 1), 8-byte half (col16 & 1); stored
    // at chunk 2*(dt ^ (sv >> 1)) + (h ^ (sv & 1))
    const int rv = kg * 4 + (col16 >> 2);
    const int sv = prefix_swz(rv);
    const int sv1 = sv >> 1;
    const int vcol = rv * D + 8 * (((col16 & 3) >> 1) ^ (sv & 1)) + 4 * (col16 & 1);  // bf16 elements

    // products of the tile at tb held in C, while the next tile loads into N
    auto step = [&](int tb, const PrefixDmaBuf& C, PrefixDmaBuf& N) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the tile are in LDS
        __syncthreads();                // ... and every wave's; N is no longer read
        if (tb + kTile < t_end) issue(tb + kTile, N);  // in flight during the products
        const uint4* kb = C.k;
        const uint16_t* vb = reinterpret_cast<const uint16_t*>(C.v);
#pragma unroll 1
        for (int half = 0; half < kTile / 64; ++half) {
            const int hb = tb + half * 64;
            if (!(active && hb < t_end && (myhalf < 0 || myhalf == half))) continue;
            floatx4 acc[4];
            float mt = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) acc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint4* kr = kb + (half * 64) * kCh + kcol + 4 * (kk ^ sk2);
#pragma unroll
                for (int k0 = 0; k0 < 4; k0 += 2) {
                    bf16x8 ka[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        ka[u] = *reinterpret_cast<const bf16x8*>(kr + (k0 + u) * 16 * kCh);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acc[k0 + u] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qv[kk], acc[k0 + u], 0, 0, 0);
                }
            }
            if (hb + 64 <= t_end) {  // every key of the half is in the chunk
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[kt][e] *= p.scale_log2;
                        mt = fmaxf(mt, acc[kt][e]);
                    }
            } else {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = hb + kt * 16 + kg * 4 + e;
                        acc[kt][e] = (t < t_end) ? acc[kt][e] * p.scale_log2 : -INFINITY;
                        mt = fmaxf(mt, acc[kt][e]);
                    }
            }
            mt = colmax4(mt);
            const float mnew = fmaxf(mrun, mt);   // finite: every half computed has a valid key
            // no column of the tile raised its running max: alpha is exactly 1
            // on every lane and the rescale of O is skipped
            const bool grew = __ballot(mt > mrun) != 0;
            const float alpha = grew ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
            float ps = 0.0f;
            shortx4 pb[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(acc[kt][e] - mnew);
                    ps += pe;
                    pb[kt][e] = static_cast<short>(f32_to_bf16(pe));
                }
            lrun = lrun * alpha + ps;
            mrun = mnew;
            if (grew) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            }
            // O^T += V^T P^T over 32 keys per product (v_mfma_f32_16x16x32_bf16):
            // key tiles kt and kt+1 form the K dimension, lane group kg
            // supplying keys kt*16 + kg*4 + 0..3 then (kt+1)*16 + kg*4 + 0..3 on
            // both operands (the same order, so every key is summed once)
#pragma unroll
            for (int kt = 0; kt < 4; kt += 2) {
                const uint16_t* vr0 = vb + (half * 64 + kt * 16) * D + vcol;
                const uint16_t* vr1 = vr0 + 16 * D;
                const bf16x8 pk = __builtin_bit_cast(
                    bf16x8, (shortx8{pb[kt][0], pb[kt][1], pb[kt][2], pb[kt][3], pb[kt + 1][0], pb[kt + 1][1],
                                     pb[kt + 1][2], pb[kt + 1][3]}));
#pragma unroll
                for (int d0 = 0; d0 < DT; d0 += 4) {
                    bf16x8 va[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const shortx4 a0 = lds_read_tr16(vr0 + 16 * ((d0 + u) ^ sv1));
                        const shortx4 a1 = lds_read_tr16(vr1 + 16 * ((d0 + u) ^ sv1));
                        va[u] = __builtin_bit_cast(bf16x8, (shortx8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}));
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        o[d0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], pk, o[d0 + u], 0, 0, 0);
                }
            }
        }
    };
    if (t_begin < t_end) issue(t_begin, SA);
    for (int tb = t_begin; tb < t_end; tb += 2 * kTile) {
        step(tb, SA, SB);
        if (tb + kTile < t_end) step(tb + kTile, SB, SA);
    }
    lrun = colsum4(lrun);
    // split pairs: the second-half wave hands (O, m, l) to the first-half wave
    // through the tile buffers, which no wave reads any more
    constexpr int kXf = DT * 4 + 2;  // floats per lane
    __syncthreads();
    const int sidx = max(tile_l - nwhole, 0);  // index of the split tile (when myhalf >= 0)
    float* xo = reinterpret_cast<float*>(sidx < 4 ? &SA : &SB) + ((sidx & 3) * 64 + lane) * kXf;
    if (active && myhalf == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) xo[dt * 4 + e] = o[dt][e];
        xo[DT * 4] = mrun;
        xo[DT * 4 + 1] = lrun;
    }
    __syncthreads();
    if (active && myhalf == 0) {
        const float m1 = xo[DT * 4], l1 = xo[DT * 4 + 1];
        const float mm = fmaxf(mrun, m1);
        const float f0 = (mrun == -INFINITY) ? 0.0f : exp2f(mrun - mm);
        const float f1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mm);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dt][e] = o[dt][e] * f0 + xo[dt * 4 + e] * f1;
        lrun = lrun * f0 + l1 * f1;
        mrun = mm;
    }
    if (active && myhalf != 1 && cg < p.NC) {
        const size_t base = (static_cast<size_t>(x) * p.Hkv + g) * p.NC + cg;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.pre_o[base * D + dt * 16 + kg * 4 + e] = o[dt][e];
        if (kg == 0) p.pre_ml[base] = make_float2(mrun, lrun);
    }
}

// ---------------------------------------------------------------- fp32 path

// mode 0: per-sequence chunks (grid.x = slot); mode 1: prefix chunks (grid.x = chunk).
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnParams p, int mode) {
    __shared__ float sc[1024];
    __shared__ float red[kThreads / 64];
    __shared__ double redd[kThreads / 64];
    __shared__ int sb, scc;
    const int tid = threadIdx.x;
    const int g = blockIdx.y, x = blockIdx.x;
    const int D = p.D;
    const size_t row_stride = static_cast<size_t>(p.Hkv) * D;
    int b = 0, t_begin, t_end, ncols, L = 0;
    int64_t kv0 = 0;
    if (mode == 0) {
        if (tid < 64) find_sequence(p, x, g, &sb, &scc);
        __syncthreads();
        b = sb;
        if (b < 0) return;
        if (scc == 0 && g == 0 && tid == 0) p.seq_base[b] = x;
        L = max(p.kv_len[b], 0);
        kv0 = p.kv_start[b];
        t_begin = scc * p.chunk;
        t_end = min(L + seq_k1(p, b), t_begin + p.chunk);
        ncols = p.G * seq_k1(p, b);
    } else {
        t_begin = x * p.prefix_chunk;
        t_end = min(p.prefix_len, t_begin + p.prefix_chunk);
        ncols = p.NC;
    }
    const int nk = t_end - t_begin;
    auto key_ptr = [&](int t, bool v) -> const float* {
        if (mode == 1)
            return (v ? p.vpf : p.kpf) + static_cast<size_t>(t) * row_stride + static_cast<size_t>(g) * D;
        return (t < L) ? (v ? p.vcf : p.kcf) + static_cast<size_t>(kv0 + t) * row_stride + static_cast<size_t>(g) * D
                       : (v ? p.vnf : p.knf) + static_cast<size_t>(seq_q0(p, b) + t - L) * row_stride + static_cast<size_t>(g) * D;
    };
    for (int col = 0; col < ncols; ++col) {
        int bb = b, cl = col;
        if (mode == 1) { bb = col / p.CPG; cl = col % p.CPG; }
        const int k1 = seq_k1(p, bb);
        if (cl >= p.G * k1) continue;  // uniform: a padding column of a shorter sequence
        const int hh = cl / k1, j = cl % k1;
        const float* qp = p.qf + (static_cast<size_t>(seq_q0(p, bb) + j) * p.Hq + g * p.G + hh) * D;
        const int lim = (mode == 1) ? t_end : min(t_end, L + j + 1);
        float lm = -INFINITY;
        for (int i = tid; i < nk; i += kThreads) {
            const int t = t_begin + i;
            float s = -INFINITY;
            if (t < lim) {
                const float* kp = key_ptr(t, false);
                float dot = 0.0f;
                for (int d = 0; d < D; ++d) dot = fmaf(qp[d], kp[d], dot);
                s = dot * p.scale_log2;
            }
            sc[i] = s;
            lm = fmaxf(lm, s);
        }
        const float m = block_max<kThreads>(lm, red);
        double ls = 0.0;
        for (int i = tid; i < nk; i += kThreads) {
            const float pe = (m == -INFINITY) ? 0.0f : exp2f(sc[i] - m);
            sc[i] = pe;
            ls += pe;
        }
        const double l = block_sum<kThreads>(ls, redd);
        __syncthreads();
        size_t base;
        float* po;
        float2* pml;
        if (mode == 0) {
            base = (static_cast<size_t>(x) * p.Hkv + g) * p.CPG + col;
            po = p.part_o; pml = p.part_ml;
        } else {
            base = (static_cast<size_t>(x) * p.Hkv + g) * p.NC + col;
            po = p.pre_o; pml = p.pre_ml;
        }
        for (int d = tid; d < D; d += kThreads) {
            float acc = 0.0f;
            for (int i = 0; i < nk; ++i)
                if (sc[i] != 0.0f) acc = fmaf(sc[i], key_ptr(t_begin + i, true)[d], acc);
            po[base * D + d] = acc;
        }
        if (tid == 0) pml[base] = make_float2(m, static_cast<float>(l));
        __syncthreads();
    }
}

// ---------------------------------------------------------------- merge

// grid: one block per (row, head); threads over the head dim.
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
    const int r = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
    int b = r / (p.K + 1);
    if (p.cu_q) {  // largest b with cu_q[b] <= r
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_q[mid] <= r) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    const int k1 = seq_k1(p, b);
    const int j = min(r - seq_q0(p, b), k1 - 1);
    const int g = h / p.G, hh = h % p.G;
    const int col = hh * k1 + j;
    const int L = max(p.kv_len[b], 0);
    int n = ceil_div(L + k1, p.chunk);
    int base = p.seq_base[b];
    // A device length above the host bound has no work items (status 3 is set
    // by the chunk kernel); keep every read inside the partial buffers.
    base = min(max(base, 0), p.slots - 1);
    n = min(n, p.slots - base);
    const size_t pcol = static_cast<size_t>(b) * p.CPG + col;

    float ms = -INFINITY;
    for (int i = 0; i < p.prefix_slots; ++i)
        ms = fmaxf(ms, p.pre_ml[(static_cast<size_t>(i) * p.Hkv + g) * p.NC + pcol].x);
    for (int i = 0; i < n; ++i)
        ms = fmaxf(ms, p.part_ml[(static_cast<size_t>(base + i) * p.Hkv + g) * p.CPG + col].x);

    for (int d = threadIdx.x; d < p.D; d += blockDim.x) {
        float acc = 0.0f, l = 0.0f;
        for (int i = 0; i < p.prefix_slots; ++i) {
            const size_t idx = (static_cast<size_t>(i) * p.Hkv + g) * p.NC + pcol;
            const float2 ml = p.pre_ml[idx];
            const float f = (ml.x == -INFINITY) ? 0.0f : exp2f(ml.x - ms);
            acc += p.pre_o[idx * p.D + d] * f;
            l += ml.y * f;
        }
        for (int i = 0; i < n; ++i) {
            const size_t idx = (static_cast<size_t>(base + i) * p.Hkv + g) * p.CPG + col;
            const float2 ml = p.part_ml[idx];
            const float f = (ml.x == -INFINITY) ? 0.0f : exp2f(ml.x - ms);
            acc += p.part_o[idx * p.D + d] * f;
            l += ml.y * f;
        }
        const float val = acc / l;
        const size_t oi = (static_cast<size_t>(r) * p.Hq + h) * p.D + d;
        if (p.bf16)
            static_cast<uint16_t*>(p.out)[oi] = f32_to_bf16(val);
        else
            static_cast<float*>(p.out)[oi] = val;
    }
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    int v = atoi(s);
    return v > 0 ? v : dflt;
}

// Decode kernel form: the multi-tile forms with 128-wide heads run column
// waves (mode 2); SPECVERIFY_ATTN_MODE=0 selects the register form for them.
int sk_mode(int D, int nct) {
    static const int env = env_int("SPECVERIFY_ATTN_MODE", 2);
    if (D != 128 || nct < 2) return 0;
    return env == 0 ? 0 : 2;
}

// Workgroups of the decode kernel that the GPU holds at once (CUs x
// resident workgroups per CU), cached per device and kernel variant.
int sk_resident_grid(int D, int nct) {
    static int cache[16][2][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 1024;  // no device: any value sizes a workspace that is never launched
    }
    int& c = cache[dev][D == 128 ? 1 : 0][nct - 1];
    if (c > 0) return c;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    const void* fn = nullptr;
#define SV_FN(DD, NN, MM) fn = reinterpret_cast<const void*>(&decode_bf16_kernel<DD, NN, MM>)
    const int mode = sk_mode(D, nct);
    if (D == 128 && mode == 2) {
        switch (nct) { case 2: SV_FN(128, 2, 2); break;
                       case 3: SV_FN(128, 3, 2); break; default: SV_FN(128, 4, 2); break; }
    } else if (D == 128) {
        switch (nct) { case 1: SV_FN(128, 1, 0); break; case 2: SV_FN(128, 2, 0); break;
                       case 3: SV_FN(128, 3, 0); break; default: SV_FN(128, 4, 0); break; }
    } else {
        switch (nct) { case 1: SV_FN(64, 1, 0); break; case 2: SV_FN(64, 2, 0); break;
                       case 3: SV_FN(64, 3, 0); break; default: SV_FN(64, 4, 0); break; }
    }
#undef SV_FN
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) per_cu = 0;
    (void)hipGetLastError();
    if (cus <= 0 || per_cu <= 0) return 1024;
    // Three resident workgroups per CU keep enough loads in flight to saturate
    // HBM; more of them only lengthen the queue that the first slice of each
    // workgroup waits in, and the last of them finish later.
    const int wpc = env_int("SPECVERIFY_SK_WGS_PER_CU", 3);
    if (wpc > 0 && wpc < per_cu) per_cu = wpc;
    c = cus * per_cu;
    return c;
}

// Workgroups of the even-split grouped-head kernel that the GPU holds at once.
int sk_stream_resident(int nct) {
    static int cache[16][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 512;  // no device: any value sizes a workspace that is never launched
    }
    int& c = cache[dev][nct - 1];
    if (c > 0) return c;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    const void* fn = nct == 2 ? reinterpret_cast<const void*>(&decode_stream_kernel<2>)
                   : nct == 3 ? reinterpret_cast<const void*>(&decode_stream_kernel<3>)
                              : reinterpret_cast<const void*>(&decode_stream_kernel<4>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) per_cu = 0;
    (void)hipGetLastError();
    if (cus <= 0 || per_cu <= 0) return 512;
    c = cus * per_cu;
    return c;
}

}  // namespace

AttnPlan attn_plan(int B, int K, int Hq, int Hkv, int D, int bf16,
                   const int32_t* kv_len_host, const int32_t* cu_q_host, int prefix_len) {
    AttnPlan pl{};
    const int K1 = K + 1;
    // keys of sequence b: its cached rows and its K_b + 1 new rows
    auto keys = [&](int b) -> long long {
        const long long L = kv_len_host[b] > 0 ? kv_len_host[b] : 0;
        return L + (cu_q_host ? cu_q_host[b + 1] - cu_q_host[b] : K1);
    };
    const size_t CPG = static_cast<size_t>(Hq / Hkv) * K1;
    const size_t NC = CPG * B;
    int pchunk = env_int("SPECVERIFY_PREFIX_CHUNK", 1024);
    pchunk = (pchunk + 63) / 64 * 64;
    if (!bf16 && pchunk > 1024) pchunk = 1024;
    // the fused merge takes at most kMergeMax parts: keep half for the prefix
    while (bf16 && prefix_len > 0 && (prefix_len + pchunk - 1) / pchunk > kMergeMax / 2)
        pchunk *= 2;
    const int pslots = prefix_len > 0 ? (prefix_len + pchunk - 1) / pchunk : 0;
    pl.ok = true;
    long long slots = 0;
    int chunk = 64;
    if (bf16) {
        // slices per sequence for the host bound
        int smax = 1;
        for (int b = 0; b < B; ++b) {
            if (keys(b) > kSkMaxKeys) pl.ok = false;
            const int sb = static_cast<int>((std::min<long long>(keys(b), kSkMaxKeys) + 15) / 16);
            smax = sb > smax ? sb : smax;
        }
        if (B > kSkMaxB) pl.ok = false;
        auto items_for = [&](int lam) {
            long long n = 0;
            for (int b = 0; b < B; ++b)
                n += ((std::min<long long>(keys(b), kSkMaxKeys) + 15) / 16 + lam - 1) / lam;
            return n * Hkv;
        };
        const int nct_all = static_cast<int>((CPG + 15) / 16);
        pl.nct = nct_all < 4 ? nct_all : 4;
        const long long cap = static_cast<long long>(sk_resident_grid(D, pl.nct)) *
                              env_int("SPECVERIFY_SK_ROUNDS", 1);
        // smallest slice budget whose work items fit in `cap` workgroups, and
        // whose chunks per sequence fit in the merge
        // (at least kLambdaMin slices, three per wave, so that short problems
        // are not split into items whose fixed costs exceed their work)
        int lo = std::min(env_int("SPECVERIFY_SK_LAMBDA_MIN", kLambdaMin), smax), hi = smax;
        const int lam_merge = (smax + (kMergeMax - pslots) - 1) / (kMergeMax - pslots);
        if (lo < lam_merge) lo = lam_merge;
        if (hi < lo) hi = lo;
        while (lo < hi) {
            const int mid = lo + (hi - lo) / 2;
            if (items_for(mid) <= cap) hi = mid; else lo = mid + 1;
        }
        // Long problems: chunks of at most kLambdaMax slices even if that
        // takes more workgroups than fit at once (the dispatcher then starts
        // the next ones as earlier ones finish, which also balances them).
        const int lam_max = std::max(env_int("SPECVERIFY_SK_LAMBDA_MAX", kLambdaMax), lam_merge);
        if (lo > lam_max) lo = lam_max;
        const int lam_env = env_int("SPECVERIFY_SK_LAMBDA", 0);
        if (lam_env >= lo) lo = lam_env;
        const long long items = items_for(lo);
        if (items > (1LL << 30)) pl.ok = false;
        pl.lambda = lo;
        pl.grid = pl.ok ? static_cast<int>(items) : 0;
        slots = pl.ok ? items : 0;
        // the per-sequence plan for the kernel arguments
        pl.plan_nb = 0;
        if (pl.ok && B <= kAttnPlanB) {
            int qrun = 0;
            for (int b = 0; b < B; ++b) {
                const int sb = static_cast<int>((std::min<long long>(keys(b), kSkMaxKeys) + 15) / 16);
                pl.plan_q[b] = qrun;
                pl.plan_s[b] = sb;
                pl.plan_row0[b] = cu_q_host ? cu_q_host[b] : b * K1;
                qrun += (sb + lo - 1) / lo;
            }
            pl.plan_q[B] = qrun;
            pl.plan_row0[B] = cu_q_host ? cu_q_host[B] : B * K1;
            pl.plan_nb = B;
        }
        // Column waves: the even split over one round of workgroups when
        // every workgroup meets at most kPieceMax segments and every segment
        // fits in the merge (else, or with SPECVERIFY_SK_CHUNKS=1, the
        // per-sequence chunks above).
        pl.plan_W = 0;
        pl.plan_N = 0;
        if (pl.plan_nb > 0 && sk_mode(D, pl.nct) == 2 && env_int("SPECVERIFY_SK_CHUNKS", 0) == 0) {
            // 32-key items per sequence for the host bound
            std::vector<int> s32(B);
            long long N = 0;  // items of all sequences, one kv head
            for (int b = 0; b < B; ++b) {
                s32[b] = static_cast<int>((std::min<long long>(keys(b), kSkMaxKeys) + 31) / 32);
                N += s32[b];
            }
            const long long Wl = std::min<long long>(sk_stream_resident(pl.nct) / Hkv,
                                                     std::max<long long>(1, N / (kLambdaMin / 2)));
            const int W = static_cast<int>(std::max<long long>(1, Wl));  // slice ranges
            auto owner = [&](long long x) { return static_cast<int>(((x + 1) * W - 1) / N); };
            std::vector<int> pieces(W, 0);
            bool fits = N > 0;
            long long st = 0;
            for (int b = 0; b < B && fits; ++b) {
                const int r0 = owner(st), r1 = owner(st + s32[b] - 1);
                if (r1 - r0 + 1 + pslots > kStreamMerge) fits = false;
                for (int r = r0; r <= r1 && fits; ++r)
                    if (++pieces[r] > kPieceMax) fits = false;
                st += s32[b];
            }
            if (fits) {
                long long run = 0;
                for (int b = 0; b < B; ++b) {
                    pl.plan_q[b] = static_cast<int>(run);
                    pl.plan_s[b] = s32[b];
                    run += s32[b];
                }
                pl.plan_q[B] = static_cast<int>(run);
                pl.plan_W = W;
                pl.plan_N = N;
                pl.grid = W * Hkv;
                slots = (static_cast<long long>(W) + B) * Hkv;
            }
        }
    } else {
        chunk = env_int("SPECVERIFY_ATTN_CHUNK", 0);
        if (chunk <= 0) {
            // largest power-of-two chunk (64..1024) that still gives >= 4 work items per CU
            chunk = 64;
            for (int c = 1024; c >= 64; c >>= 1) {
                long long items = 0;
                for (int b = 0; b < B; ++b) items += (keys(b) + c - 1) / c;
                if (items * Hkv >= 1024) { chunk = c; break; }
            }
        }
        chunk = (chunk + 63) / 64 * 64;
        if (chunk > 1024) chunk = 1024;
        for (int b = 0; b < B; ++b) slots += (keys(b) + chunk - 1) / chunk;
        if (slots > (1LL << 30)) pl.ok = false;
        slots *= Hkv;  // the fp32 partials are per (slot, kv head)
    }
    // The arrival counters come first: their place depends on B and Hkv only,
    // so calls with other lengths or draft counts never put data over them.
    pl.counter_bytes = (static_cast<size_t>(B) * Hkv * 4 + 255) & ~static_cast<size_t>(255);
    size_t off = pl.counter_bytes;
    auto take = [&](size_t n) { off = (off + 255) & ~static_cast<size_t>(255); off += n; };
    take(static_cast<size_t>(B) * 4);
    take(static_cast<size_t>(slots) * CPG * D * 4);
    take(static_cast<size_t>(slots) * CPG * 8);
    take(static_cast<size_t>(pslots) * Hkv * NC * D * 4);
    take(static_cast<size_t>(pslots) * Hkv * NC * 8);
    pl.chunk = chunk;
    pl.prefix_chunk = pchunk;
    pl.slots = bf16 ? static_cast<int>(slots) : static_cast<int>(slots / (Hkv > 0 ? Hkv : 1));
    pl.prefix_slots = pslots;
    pl.bytes = (off + 255) & ~static_cast<size_t>(255);
    return pl;
}

hipError_t attn_launch(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
    AttnParams p{};
    p.q = static_cast<const uint16_t*>(a.q);
    p.k_cache = static_cast<const uint16_t*>(a.k_cache);
    p.v_cache = static_cast<const uint16_t*>(a.v_cache);
    p.k_new = static_cast<const uint16_t*>(a.k_new);
    p.v_new = static_cast<const uint16_t*>(a.v_new);
    p.k_prefix = static_cast<const uint16_t*>(a.k_prefix);
    p.v_prefix = static_cast<const uint16_t*>(a.v_prefix);
    p.qf = static_cast<const float*>(a.q);
    p.kcf = static_cast<const float*>(a.k_cache);
    p.vcf = static_cast<const float*>(a.v_cache);
    p.knf = static_cast<const float*>(a.k_new);
    p.vnf = static_cast<const float*>(a.v_new);
    p.kpf = static_cast<const float*>(a.k_prefix);
    p.vpf = static_cast<const float*>(a.v_prefix);
    p.kv_start = a.kv_start;
    p.kv_len = a.kv_len;
    p.out = a.out;
    p.status = a.status;
    p.cu_q = a.cu_q;
    p.rows = a.rows;
    p.B = a.B;
    p.K = a.K;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.CPG = p.G * (a.K + 1);
    p.NC = p.CPG * a.B;
    p.D = a.D;
    p.chunk = pl.chunk;
    p.prefix_chunk = pl.prefix_chunk;
    p.prefix_len = a.prefix_len;
    p.prefix_slots = pl.prefix_slots;
    p.slots = pl.slots;
    p.lambda = pl.lambda;
    p.bf16 = a.bf16;
    p.xcd = env_int("SPECVERIFY_ATTN_XCD", 0) > 0 ? 1 : 0;
    p.scale_log2 = a.scale * kLog2e;

    // counters, then the data region (its layout as in attn_plan)
    char* base = static_cast<char*>(a.workspace);
    if (a.counters) {
        p.merge_cnt = static_cast<int*>(a.counters);
    } else {
        p.merge_cnt = reinterpret_cast<int*>(base);
        base += pl.counter_bytes;
    }
    size_t off = 0;
    auto take = [&](size_t n) {
        off = (off + 255) & ~static_cast<size_t>(255);
        char* r = base + off;
        off += n;
        return r;
    };
    const size_t CPG = p.CPG, NC = p.NC;
    const size_t pslots_all = a.bf16 ? static_cast<size_t>(pl.slots) : static_cast<size_t>(pl.slots) * a.Hkv;
    p.seq_base = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * 4));
    p.part_o = reinterpret_cast<float*>(take(pslots_all * CPG * a.D * 4));
    p.part_ml = reinterpret_cast<float2*>(take(pslots_all * CPG * 8));
    p.pre_o = reinterpret_cast<float*>(take(static_cast<size_t>(pl.prefix_slots) * a.Hkv * NC * a.D * 4));
    p.pre_ml = reinterpret_cast<float2*>(take(static_cast<size_t>(pl.prefix_slots) * a.Hkv * NC * 8));

    if (a.bf16) {
        if (pl.prefix_slots > 0) {
            const int tiles = (p.NC + 15) / 16;
            const int groups = (tiles + 15) / 16;
            dim3 grid(pl.prefix_slots, a.Hkv, groups);  // 16 waves: all load, the group's tiles compute
            if (a.D == 128)
                hipLaunchKernelGGL(prefix_dma_kernel, grid, dim3(1024), 0, stream, p);
            else
                hipLaunchKernelGGL(prefix_bf16_kernel<64>, grid, dim3(1024), 0, stream, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int nct = pl.nct;
        DecPlan dp;
        dp.nb = pl.plan_nb;
        dp.W = pl.plan_W;
        dp.N = pl.plan_N;
        for (int b = 0; b <= pl.plan_nb && pl.plan_nb > 0; ++b) {
            dp.q[b] = pl.plan_q[b];
            dp.row0[b] = pl.plan_row0[b];
            if (b < pl.plan_nb) dp.s[b] = pl.plan_s[b];
        }
        // XCD-contiguous items need a grid that is a multiple of 8 (the extra
        // workgroups find no item and leave)
        dim3 grid(p.xcd ? (pl.grid + 7) / 8 * 8 : pl.grid);
        // With timing events, the dispatch itself stamps them at the kernel's
        // start and end (the same timestamps a kernel trace reports).
#define SV_DECODE(DD, NN, RR)                                                                      \
    do {                                                                                           \
        if (a.ev_start && a.ev_stop)                                                               \
            hipExtLaunchKernelGGL((decode_bf16_kernel<DD, NN, RR>), grid, dim3(kThreads), 0,      \
                                  stream, a.ev_start, a.ev_stop, 0, p, dp);                        \
        else                                                                                       \
            hipLaunchKernelGGL((decode_bf16_kernel<DD, NN, RR>), grid, dim3(kThreads), 0, stream, \
                               p, dp);                                                             \
    } while (0)
        const int mode = sk_mode(a.D, nct);
        if (pl.plan_W > 0) {
            dim3 sgrid(pl.plan_W * a.Hkv);
#define SV_STREAM(NN)                                                                              \
    do {                                                                                           \
        if (a.ev_start && a.ev_stop)                                                               \
            hipExtLaunchKernelGGL((decode_stream_kernel<NN>), sgrid, dim3(kThreads), 0, stream,    \
                                  a.ev_start, a.ev_stop, 0, p, dp);                                \
        else                                                                                       \
            hipLaunchKernelGGL((decode_stream_kernel<NN>), sgrid, dim3(kThreads), 0, stream, p, dp); \
    } while (0)
            switch (nct) {
                case 2: SV_STREAM(2); break;
                case 3: SV_STREAM(3); break;
                default: SV_STREAM(4); break;
            }
#undef SV_STREAM
        } else if (a.D == 128 && mode == 2) {
            switch (nct) {
                case 2: SV_DECODE(128, 2, 2); break;
                case 3: SV_DECODE(128, 3, 2); break;
                default: SV_DECODE(128, 4, 2); break;
            }
        } else if (a.D == 128) {
            switch (nct) {
                case 1: SV_DECODE(128, 1, 0); break;
                case 2: SV_DECODE(128, 2, 0); break;
                case 3: SV_DECODE(128, 3, 0); break;
                default: SV_DECODE(128, 4, 0); break;
            }
        } else {
            switch (nct) {
                case 1: SV_DECODE(64, 1, 0); break;
                case 2: SV_DECODE(64, 2, 0); break;
                case 3: SV_DECODE(64, 3, 0); break;
                default: SV_DECODE(64, 4, 0); break;
            }
        }
#undef SV_DECODE
    } else {
        if (pl.prefix_slots > 0) {
            hipLaunchKernelGGL(attn_f32_kernel, dim3(pl.prefix_slots, a.Hkv), dim3(kThreads), 0,
                               stream, p, 1);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (a.ev_start && a.ev_stop)
            hipExtLaunchKernelGGL(attn_f32_kernel, dim3(pl.slots, a.Hkv), dim3(kThreads), 0, stream,
                                  a.ev_start, a.ev_stop, 0, p, 0);
        else
            hipLaunchKernelGGL(attn_f32_kernel, dim3(pl.slots, a.Hkv), dim3(kThreads), 0, stream, p,
                               0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.bf16) return hipSuccess;  // the chunk kernel merges in its last workgroup
    const int mthreads = a.D <= 64 ? 64 : (a.D <= 128 ? 128 : 256);
    hipLaunchKernelGGL(merge_kernel, dim3(a.rows * a.Hq), dim3(mthreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace sv
