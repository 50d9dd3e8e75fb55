// Modified rejection sampling for a batch of verify rounds on gfx950.
//
// Method: "Accelerating Large Language Model Decoding with Speculative
// Sampling", section "Modified rejection sampling" and Theorem 1: accept draft
// x_j with probability min(1, q(x_j)/p(x_j)) left to right, resample the first
// rejected position from (q - p)_+, draw a bonus token from the last target
// row when all K drafts pass; temperature and nucleus modify q and p first.
//
// rows_kernel  grid = rows x segments of 4096 logits; one kernel for the whole
//   round when the nucleus is on (or greedy), chained by last-arriver counters:
//   segment  read the segment once: max, fp64 mass relative to it, and
//            (nucleus) the segment's candidate list: every element of the
//            highest quarter-unit bins of z/T, as many bins as fit in 256
//            entries, stored in id order.  A nucleus of top_p < 1 keeps the
//            upper part of the distribution, so the lists normally hold it
//            whole.
//   row      the last segment of a row merges it: max, normaliser, fp64
//            masses of the listed entries over 1/16-unit bins, and the exact
//            tie-closed nucleus threshold (the boundary bin from the bin
//            masses, then its few entries ranked exactly).  When a list
//            misses part of the nucleus the row falls back to a radix select
//            over the whole row.
//   sequence the last row of a sequence runs the accept scan and draws the
//            emitted token from the stopping row's lists: the residual
//            (q' - p')_+ and q' vanish outside the target nucleus, so the
//            draft logits are read at the target nucleus members' ids only.
//            A row without a complete list is drawn by a pass over the
//            whole row.
// draw_kernel  (no nucleus) grid = sequences x segments: fp64 residual or
//   bonus weights of the stopping row, per-segment sums; the last segment
//   picks the crossing segment and scans it exactly.
// Every quantity that decides a token is fp64; the exp of the logits is the
// table-driven fp64 exp of sv_math.h (table of 2^(j/64) built per workgroup).
// A chain of dependent global accesses costs about a microsecond per link
// under load, so every merge issues its loads together.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_math.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kSeg = kThreads * kPerThread;  // 4096 logits per segment
constexpr int kFine = 4;                     // row bins per segment bin
constexpr int kBins = 512;                   // 1/16-unit bins of z/T below the row max (32 units)
constexpr int kBinsPerLane = kBins / 64;
constexpr int kCutBins = 64;                 // quarter-unit bins below the segment max a list may span
constexpr int kList = kThreads;              // candidate list capacity per segment
constexpr int kCap = 1024;                   // boundary-bin entries ranked in LDS
constexpr int kMaxSeg = 64;                  // V <= 64 * 4096
constexpr int kChunk = 16;                   // list segments a thread loads per round trip
constexpr int kMaxRowsPerSeq = 2 * 64 + 1;   // K <= 64

struct SegHead {
    float m;      // segment max (greedy: max value)
    int kb_top;   // row bin of the max (greedy: index of the max)
    int kb_cut;   // nucleus: every element with row bin >= kb_cut is in the list
    int n;        // nucleus: list length
    double S;     // sum of exp((z - m)/T) over the segment
};

struct RowRec {
    float m;      // row max
    float tau;    // nucleus threshold logit (-inf: no nucleus)
    double S;     // kept mass relative to m (= full normaliser without nucleus)
    double wx;    // exp((z[x] - m)/T) for the drafted token x of this row
    int kept;     // drafted token inside the nucleus
    int argmax;   // lowest id of the row maximum (greedy)
    int fast;     // the row's lists hold its whole nucleus
    int pad;
};

struct SeqRec {
    int n;        // accepted drafts
    int pad;
};

struct AcceptParams {
    const void* target;
    const void* draft;
    const int32_t* draft_tokens;
    const float* u_accept;
    const float* u_sample;
    int32_t* n_accepted;
    int32_t* out_tokens;
    int32_t* status;
    SegHead* seg;
    unsigned long long* list;  // [nrows][nseg][kList]: (id << 32) | bits of z, ids ascending
    RowRec* rows;
    float* zx;                 // [nrows]: logit of the row's drafted token (segment that holds it)
    SeqRec* seqs;
    double* dsum;
    double* qsum;
    int* row_cnt;
    int* seq_cnt;
    int* draw_cnt;
    const int32_t* cu_q;       // [B+1] ragged draft lengths: target rows of b start at cu_q[b]
    int nt;                    // target rows (cu_q[B], or B*(K+1))
    int B, K, V, nseg, nrows, grid_rows;  // K: the largest draft length
    int bf16, vec, nucleus, greedy;  // nucleus: a filter is on (top_p < 1 or top_k)
    int top_k;                       // keep the k largest logits and their ties (0: off)
    double invT;
    double top_p;
    float bscale;    // 16 / T: row bin of z is floor(z * bscale)
    float bscale_c;  // 4 / T: segment bin of z is floor(z * bscale_c); row bin = 4 * segment bin + 0..3
};

// Sequence b owns target rows q0 .. q0+K_b (q0 = cu_q[b], or b*(K+1)) and draft
// rows nt+q0-b .. nt+q0-b+K_b-1; its drafts and accept uniforms start at
// q0-b, its output tokens at q0.
__device__ __forceinline__ int seq_q0(const AcceptParams& p, int b) {
    return p.cu_q ? p.cu_q[b] : b * (p.K + 1);
}
__device__ __forceinline__ int seq_kb(const AcceptParams& p, int b) {
    return p.cu_q ? min(max(p.cu_q[b + 1] - p.cu_q[b] - 1, 0), p.K) : p.K;
}

// ---------------------------------------------------------------- loads

__device__ __forceinline__ float load1(const void* row, int bf16, int e) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(row)[e])
                : static_cast<const float*>(row)[e];
}

// Four consecutive logits starting at e (e % 4 == 0); -inf past V.
__device__ __forceinline__ void load4(const void* row, int bf16, int vec, int V, int e,
                                      float* z) {
    if (vec && e + 3 < V) {
        if (bf16) {
            uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + e);
            z[0] = __uint_as_float(u.x << 16);
            z[1] = __uint_as_float(u.x & 0xFFFF0000u);
            z[2] = __uint_as_float(u.y << 16);
            z[3] = __uint_as_float(u.y & 0xFFFF0000u);
        } else {
            float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + e);
            z[0] = f.x; z[1] = f.y; z[2] = f.z; z[3] = f.w;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] = (e + k < V) ? load1(row, bf16, e + k) : -INFINITY;
}

// Segment element k of thread tid: index seg*4096 + (k/4)*1024 + tid*4 + k%4.
__device__ __forceinline__ void load_segment(const void* row, int bf16, int vec, int V,
                                             int s, int tid, float* z) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        load4(row, bf16, vec, V, s * kSeg + i * 1024 + tid * 4, z + 4 * i);
}

__device__ __forceinline__ int seg_index(int s, int tid, int k) {
    return s * kSeg + (k >> 2) * 1024 + tid * 4 + (k & 3);
}

__device__ __forceinline__ const void* row_ptr(const AcceptParams& p, int r) {
    const int nt = p.nt;
    const size_t es = p.bf16 ? 2 : 4;
    if (r < nt) return static_cast<const char*>(p.target) + static_cast<size_t>(r) * p.V * es;
    return static_cast<const char*>(p.draft) + static_cast<size_t>(r - nt) * p.V * es;
}

__device__ __forceinline__ int bin_of(float z, float bscale) {
    float y = fminf(fmaxf(z * bscale, -1.0e9f), 1.0e9f);
    return static_cast<int>(floorf(y));
}

// fp64 weight of logit z relative to the max m (both exact in double).
__device__ __forceinline__ double weight(float z, float m, double invT, const double* tab) {
    return exp_nonpos((static_cast<double>(z) - static_cast<double>(m)) * invT, tab);
}

// Fill the 64-entry table 2^(j/64) of exp_nonpos (threads 0..63); the caller
// synchronises before use.
__device__ __forceinline__ void fill_exp_table(double* tab) {
    if (threadIdx.x < 64) tab[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) * (1.0 / 64.0));
}

// Order-preserving 32-bit key of a float (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t fkey(float z) {
    uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------- LDS layout

struct RowsLds {
    double tab[64];           // 2^(j/64) for exp_nonpos
    double red_d[kThreads / 64];
    double red_d2[kThreads / 64];
    float red_f[kThreads / 64];
    int flag;
    union alignas(16) {
        struct {              // segment: per-wave counts of bins kb_top - o
            int hc[4][kCutBins];
            int fit;
            unsigned long long wtot[kThreads / 64];
        } seg;
        struct {              // row merge: bin masses, boundary-bin entries
            double hm[kBins];         // row mass per bin kb_top - og
            int hcnt[kBins];          // row count per bin (top-k)
            unsigned long long ck[kCap + 8];  // order key: (z desc, id asc) <-> key desc
            int wcnt[kThreads / 64];
            float rz[kCap];   // z in rank order
            double rw[kCap];  // weight in rank order
        } cand;
        struct {              // radix select fallback
            double rh_m[256];
            int rh_c[256];
        } rad;
        struct {              // sequence
            RowRec rr[kMaxRowsPerSeq];
            float ua[64];
            int x[64];
            double scan[kThreads];
            double scan2[kThreads];
            float zpa[kChunk * kThreads];     // draft logits of every run's members
        } sq;
    };
    // row merge
    float seg_m[kMaxSeg];
    int seg_kb[kMaxSeg];
    int seg_cut[kMaxSeg];
    int seg_n[kMaxSeg];
    double seg_S[kMaxSeg];
    double sc[kMaxSeg];       // per-segment rescale exp((m_s - m)/T)
    float m;
    int argmax;
    double S;
    float zx;                 // logit of the drafted token of the row
    int kb_top, kb_lo;
    float zk;                 // top-k threshold logit (-inf: no top-k)
    int fastk;                // the lists decided the top-k threshold
    double Sk;                // mass of the top-k set (the full normaliser without top-k)
    int abovec;               // radix select: count above the current digit
    int og;
    int ccount;
    int fast;
    double above;
    float tau;
    double kept;
    uint32_t prefix, mask;
    int chosen;
    int n, tok, lastpos;
    float us;                 // u_sample of the sequence
    int rb;                   // sequence of the workgroup's row (ragged draft lengths)
};

// Exact tie-closed threshold by radix select over the whole row (4 passes of
// 8 bits over order-preserving keys, fp64 digit masses and digit counts),
// among the elements with z >= zmin.  kcount > 0: the kcount-th largest value
// (top-k); else the nucleus boundary, the largest value whose tie-closed top
// set reaches `target` mass.  Sets L.tau and L.kept (mass of z >= tau, z >=
// zmin).  Used when a row's candidate lists cannot decide.
__device__ __forceinline__ void radix_threshold(const AcceptParams& p, const void* row, float m, double target,
                                int kcount, float zmin, RowsLds& L) {
    const int tid = threadIdx.x;
    if (tid == 0) { L.prefix = 0; L.mask = 0; L.above = 0.0; L.abovec = 0; }
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int d = tid; d < 256; d += kThreads) { L.rad.rh_m[d] = 0.0; L.rad.rh_c[d] = 0; }
        __syncthreads();
        const uint32_t prefix = L.prefix, mask = L.mask;
        for (int base = 0; base < p.V; base += kThreads * 16) {
            float z[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) load4(row, p.bf16, p.vec, p.V, base + (i * kThreads + tid) * 4, z + 4 * i);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int e = base + ((k >> 2) * kThreads + tid) * 4 + (k & 3);
                const uint32_t key = fkey(z[k]);
                if (e < p.V && (key & mask) == prefix && z[k] >= zmin) {
                    const int d = (key >> shift) & 0xFF;
                    atomicAdd(&L.rad.rh_m[d], weight(z[k], m, p.invT, L.tab));
                    atomicAdd(&L.rad.rh_c[d], 1);
                }
            }
        }
        __syncthreads();
        if (tid == 0) {
            double cum = L.above;
            int cumc = L.abovec;
            int chosen = -1, lowest = -1;
            for (int d = 255; d >= 0; --d) {
                if (L.rad.rh_c[d] == 0) continue;
                lowest = d;
                const bool hit = kcount > 0 ? (cumc + L.rad.rh_c[d] >= kcount)
                                            : (cum + L.rad.rh_m[d] >= target);
                if (hit) { chosen = d; break; }
                cum += L.rad.rh_m[d];
                cumc += L.rad.rh_c[d];
            }
            if (chosen < 0) {  // rounding left the target unreached: keep everything
                chosen = lowest;
                cum -= L.rad.rh_m[lowest];
                cumc -= L.rad.rh_c[lowest];
            }
            L.above = cum;
            L.abovec = cumc;
            L.prefix |= static_cast<uint32_t>(chosen) << shift;
            L.mask |= 0xFFu << shift;
            L.chosen = chosen;
        }
        __syncthreads();
    }
    if (tid == 0) {
        L.tau = fkey_inv(L.prefix);
        L.kept = L.above + L.rad.rh_m[L.chosen];
    }
    __syncthreads();
}

// Block-wide exclusive scan of one double per thread in thread order; returns
// the exclusive prefix and writes the total to *total.  Fixed order.
__device__ __forceinline__ double block_excl_scan(double v, double* scan, double* total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const double inc = wave_incl_scan(v, lane);
    __syncthreads();
    scan[tid] = inc;
    __syncthreads();
    double off = 0.0, tot = 0.0;
#pragma unroll
    for (int u = 0; u < kThreads / 64; ++u) {
        const double t = scan[u * 64 + 63];
        if (u < wv) off += t;
        tot += t;
    }
    *total = tot;
    return off + inc - v;
}

// Two block-wide exclusive scans at once (thread order, fixed order).
__device__ __forceinline__ void block_excl_scan2(double a, double b, double* sa, double* sb,
                                                 double* ea, double* eb, double* ta, double* tb) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const double ia = wave_incl_scan(a, lane);
    const double ib = wave_incl_scan(b, lane);
    __syncthreads();
    sa[tid] = ia;
    sb[tid] = ib;
    __syncthreads();
    double oa = 0.0, ob = 0.0, xa = 0.0, xb = 0.0;
#pragma unroll
    for (int u = 0; u < kThreads / 64; ++u) {
        const double va = sa[u * 64 + 63], vb = sb[u * 64 + 63];
        if (u < wv) { oa += va; ob += vb; }
        xa += va;
        xb += vb;
    }
    *ta = xa;
    *tb = xb;
    *ea = oa + ia - a;
    *eb = ob + ib - b;
}

// ---------------------------------------------------------------- segment

// Counts of bins kb_top - o, o in [0, kCutBins), and the candidate list: all
// elements of the highest bins that fit in kList entries, in id order; then
// the segment head.  The row merge takes bin masses from the lists.
__device__ __forceinline__ void segment_list(const AcceptParams& p, int r, int s, const float* z,
                                             float ms, double Ss, RowsLds& L) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int kb_top = bin_of(ms, p.bscale_c);  // segment bins
    static_assert(4 * kCutBins == kThreads, "one counter per thread");
    (&L.seg.hc[0][0])[tid] = 0;
    __syncthreads();
    int o[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        o[k] = (z[k] == -INFINITY) ? kCutBins : kb_top - bin_of(z[k], p.bscale_c);
        if (o[k] < kCutBins) atomicAdd(&L.seg.hc[wv][o[k]], 1);
    }
    __syncthreads();
    if (tid < kCutBins) {
        // cumulative counts from the top bin down; bins 0 .. fit-1 fit in the list
        const int c = (L.seg.hc[0][tid] + L.seg.hc[1][tid]) + (L.seg.hc[2][tid] + L.seg.hc[3][tid]);
        const int cum = wave_incl_scan(c, lane);
        const unsigned long long bal = __ballot(cum <= kList);
        if (lane == 0) L.seg.fit = __popcll(bal);
    }
    __syncthreads();
    // bins 0 .. ocut fit (cum is nondecreasing); -1: the top bin alone overflows
    const int ocut = L.seg.fit - 1;
    // positions in id order: group g = k/4 holds ids s*4096 + g*1024 + 4*tid + k%4
    unsigned long long packed = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
        if (o[k] <= ocut) packed += 1ull << (16 * (k >> 2));
    // 64-bit words holding four 16-bit counters: no carry crosses a field
    const unsigned long long inc = wave_incl_scan(packed, lane);
    if (lane == 63) L.seg.wtot[wv] = inc;
    __syncthreads();
    unsigned long long off = 0, tot = 0;
#pragma unroll
    for (int u = 0; u < kThreads / 64; ++u) {
        if (u < wv) off += L.seg.wtot[u];
        tot += L.seg.wtot[u];
    }
    const unsigned long long excl = off + inc - packed;
    int gofs[4];
    int run = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        gofs[g] = run + static_cast<int>((excl >> (16 * g)) & 0xFFFF);
        run += static_cast<int>((tot >> (16 * g)) & 0xFFFF);
    }
    unsigned long long* dst = p.list + (static_cast<size_t>(r) * p.nseg + s) * kList;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        if (o[k] <= ocut) {
            const int g = k >> 2;
            const unsigned id = static_cast<unsigned>(seg_index(s, tid, k));
            st_coh(dst + gofs[g], (static_cast<unsigned long long>(id) << 32) | __float_as_uint(z[k]));
            ++gofs[g];
        }
    }
    if (tid == 0) {
        SegHead* h = p.seg + static_cast<size_t>(r) * p.nseg + s;
        st_coh(&h->m, ms);
        st_coh(&h->kb_top, bin_of(ms, p.bscale));
        // segment bin c covers row bins kFine*c .. kFine*c + kFine-1 (the scales
        // differ by a power of two, so both floors agree)
        st_coh(&h->kb_cut, kFine * (kb_top - ocut));
        st_coh(&h->n, run);
        st_coh(&h->S, Ss);
    }
}

// ---------------------------------------------------------------- row merge

__device__ __forceinline__ float entry_z(unsigned long long e) {
    return __uint_as_float(static_cast<unsigned>(e));
}
__device__ __forceinline__ int entry_id(unsigned long long e) { return static_cast<int>(e >> 32); }

// Gather the listed entries of bin kb_sel with z >= zmin (held in registers:
// slot tid of segments 0..kChunk-1) and rank them by (z desc, id asc):
// L.cand.rz[rank] = z, L.cand.rw[rank] = its fp64 weight relative to the row
// max m, L.ccount = their number.  Returns false in every thread
// when there are none or more than kCap.
__device__ __forceinline__ bool rank_bin(const AcceptParams& p, const unsigned long long* e, int kb_sel,
                                         float zmin, float m, RowsLds& L) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // per-wave counts, one barrier for the wave offsets, then positions from
    // the ballots (no contended counter)
    unsigned long long bal[kChunk];
    int wcount = 0;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
        const float zc = entry_z(e[c]);
        const bool in = static_cast<int>(c < p.nseg) & static_cast<int>(tid < L.seg_n[min(c, p.nseg - 1)]) &
                        static_cast<int>(bin_of(zc, p.bscale) == kb_sel) & static_cast<int>(zc >= zmin);
        bal[c] = __ballot(in);
        wcount += __popcll(bal[c]);
    }
    // (earlier reads of wcnt, ccount, ck, rz and rw all end before barriers of
    // the caller)
    if (lane == 0) L.cand.wcnt[wv] = wcount;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int u = 0; u < kThreads / 64; ++u) base += (u < wv) ? L.cand.wcnt[u] : 0;
    const int n = L.cand.wcnt[0] + L.cand.wcnt[1] + L.cand.wcnt[2] + L.cand.wcnt[3];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
        const unsigned long long bc = bal[c];
        const int slot = base + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bc >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bc), 0));
        if (((bc >> lane) & 1ull) && slot < kCap) {
            const uint32_t id = static_cast<uint32_t>(entry_id(e[c]));
            L.cand.ck[slot] = (static_cast<unsigned long long>(fkey(entry_z(e[c]))) << 32) | (0xFFFFFFFFu - id);
        }
        base += __popcll(bc);
    }
    if (tid == 0) L.ccount = n;
    if (n > kCap || n == 0) {
        __syncthreads();
        return false;
    }
    // rank = number of larger keys (keys are distinct); every lane of a wave
    // reads the same keys (LDS broadcast), 8 per batch
    for (int i = n + tid; i < ((n + 7) & ~7); i += kThreads) L.cand.ck[i] = 0ull;  // pad: never larger
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const unsigned long long ki = L.cand.ck[i];
        int rank = 0;
        const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(L.cand.ck);
#pragma unroll 2
        for (int j = 0; j < n; j += 8) {
            const ulonglong2 a0 = k2[j / 2], a1 = k2[j / 2 + 1], a2 = k2[j / 2 + 2], a3 = k2[j / 2 + 3];
            rank += static_cast<int>(a0.x > ki) + static_cast<int>(a0.y > ki) + static_cast<int>(a1.x > ki) +
                    static_cast<int>(a1.y > ki) + static_cast<int>(a2.x > ki) + static_cast<int>(a2.y > ki) +
                    static_cast<int>(a3.x > ki) + static_cast<int>(a3.y > ki);
        }
        const float zi = fkey_inv(static_cast<uint32_t>(ki >> 32));
        L.cand.rz[rank] = zi;
        L.cand.rw[rank] = weight(zi, m, p.invT, L.tab);  // relative to the row max
    }
    __syncthreads();
    return true;
}

// Exact tie-closed nucleus threshold of a row from its merged bin masses (L.hm,
// fp64, entries with z >= zmin) and the boundary bin's listed entries.  Sets
// L.fast = 0 when the lists cannot decide it.
__device__ __forceinline__ void list_threshold(const AcceptParams& p, double target, float zmin,
                                               const unsigned long long* e, RowsLds& L) {
    const int tid = threadIdx.x;
    const float m = L.m;
    const int kb_top = L.kb_top;
    if (tid < 64) {
        // first bin whose cumulative mass from the top reaches the target
        // (lane l: bins kBinsPerLane*l .. +kBinsPerLane-1)
        const int lane = tid;
        double v[kBinsPerLane], tot = 0.0;
#pragma unroll
        for (int i = 0; i < kBinsPerLane; ++i) {
            v[i] = L.cand.hm[kBinsPerLane * lane + i];
            tot += v[i];
        }
        const double inc = wave_incl_scan(tot, lane);
        const double before = inc - tot;
        const unsigned long long hit = __ballot(inc >= target);
        int og = -1;
        double cum = 0.0;
        if (hit) {
            const int l = __ffsll(hit) - 1;
            double run = __shfl(before, l, 64);
            // the hitting lane's bins in order, from its prefix (read back
            // from LDS: independent broadcast reads, not a chain of shuffles)
            double vl[kBinsPerLane];
#pragma unroll
            for (int i = 0; i < kBinsPerLane; ++i) vl[i] = L.cand.hm[kBinsPerLane * l + i];
            int sel = kBinsPerLane - 1;
            double at = 0.0;
            bool found = false;
#pragma unroll
            for (int i = 0; i < kBinsPerLane; ++i) {
                const double vi = vl[i];
                if (!found && run + vi >= target) { sel = i; at = run; found = true; }
                run += vi;
            }
            if (!found) at = run - vl[kBinsPerLane - 1];
            og = kBinsPerLane * l + sel;
            cum = at;
        }
        if (lane == 0) {
            // the boundary bin must be complete in every segment's list
            const bool ok = og >= 0 && kb_top - og >= L.kb_lo && p.nseg <= kChunk;
            L.og = og;
            L.above = cum;
            L.fast = ok ? 1 : 0;
        }
    }
    __syncthreads();
    if (!L.fast) return;
    if (!rank_bin(p, e, kb_top - L.og, zmin, m, L)) {
        if (tid == 0) L.fast = 0;
        __syncthreads();
        return;
    }
    const int n = L.ccount;
    if (tid < 64) {
        const int lane = tid;
        double run = L.above;
        int istar = -1;
        for (int c0 = 0; c0 < n && istar < 0; c0 += 64) {
            const double v = (c0 + lane < n) ? L.cand.rw[c0 + lane] : 0.0;
            const double inc = run + wave_incl_scan(v, lane);
            const unsigned long long hit = __ballot(c0 + lane < n && inc >= target);
            if (hit) istar = c0 + __ffsll(hit) - 1;
            run = __shfl(inc, 63, 64);
        }
        if (istar < 0) istar = n - 1;
        const float tau = L.cand.rz[istar];
        // kept mass: everything above the bin plus the entries >= tau (ties kept)
        double part = 0.0;
        for (int c0 = 0; c0 < n; c0 += 64) {
            const int i = c0 + lane;
            part += (i < n && L.cand.rz[i] >= tau) ? L.cand.rw[i] : 0.0;
        }
        part = wave_sum(part);
        if (lane == 0) {
            L.tau = tau;
            L.kept = L.above + part;
        }
    }
    __syncthreads();
}

// Top-k threshold of a row from its merged bin counts (L.hcnt) and the
// boundary bin's listed entries: the k-th largest logit (ties kept).  Sets
// L.zk, and L.fastk = 0 when the lists cannot decide it.
__device__ __forceinline__ void topk_lists(const AcceptParams& p, const unsigned long long* e, RowsLds& L) {
    const int tid = threadIdx.x;
    const int kb_top = L.kb_top;
    if (tid < 64) {
        const int lane = tid;
        int cv[kBinsPerLane], tot = 0;
#pragma unroll
        for (int i = 0; i < kBinsPerLane; ++i) {
            cv[i] = L.cand.hcnt[kBinsPerLane * lane + i];
            tot += cv[i];
        }
        const int inc = wave_incl_scan(tot, lane);
        const int before = inc - tot;
        const unsigned long long hit = __ballot(inc >= p.top_k);
        int og = -1, cum = 0;
        if (hit) {
            const int l = __ffsll(hit) - 1;
            int run = __shfl(before, l, 64);
            int cl[kBinsPerLane];
#pragma unroll
            for (int i = 0; i < kBinsPerLane; ++i) cl[i] = L.cand.hcnt[kBinsPerLane * l + i];
            int sel = kBinsPerLane - 1, at = 0;
            bool found = false;
#pragma unroll
            for (int i = 0; i < kBinsPerLane; ++i) {
                const int ci = cl[i];
                if (!found && run + ci >= p.top_k) { sel = i; at = run; found = true; }
                run += ci;
            }
            if (!found) at = run - cl[kBinsPerLane - 1];
            og = kBinsPerLane * l + sel;
            cum = at;
        }
        if (lane == 0) {
            const bool ok = og >= 0 && kb_top - og >= L.kb_lo && p.nseg <= kChunk;
            L.og = og;
            L.abovec = cum;
            L.fastk = ok ? 1 : 0;
        }
    }
    __syncthreads();
    if (!L.fastk) return;
    if (!rank_bin(p, e, kb_top - L.og, -INFINITY, L.m, L)) {
        if (tid == 0) L.fastk = 0;
        __syncthreads();
        return;
    }
    if (tid == 0) L.zk = L.cand.rz[min(p.top_k - L.abovec - 1, L.ccount - 1)];
    __syncthreads();
}

// Merge the segments of row r and write its RowRec.
__device__ __forceinline__ void finalize_row(const AcceptParams& p, int r, int b, RowsLds& L) {
    const int tid = threadIdx.x;
    const void* row = row_ptr(p, r);
    const SegHead* sr = p.seg + static_cast<size_t>(r) * p.nseg;

    // drafted token of this row: target row j < K_b (draft index r - b), or
    // draft row j (draft index r - nt); -1: the bonus row
    const bool is_target = r < p.nt;
    const int xi = is_target ? ((r + 1 < seq_q0(p, b + 1)) ? r - b : -1) : r - p.nt;
    const int j = xi;  // >= 0 iff the row has a drafted token

    // one round trip: segment heads, the first kChunk segments' list slot
    // tid, and the drafted logit
    if (tid < p.nseg) {
        L.seg_m[tid] = ld_coh(&sr[tid].m);
        L.seg_kb[tid] = ld_coh(&sr[tid].kb_top);
        L.seg_cut[tid] = ld_coh(&sr[tid].kb_cut);
        L.seg_n[tid] = ld_coh(&sr[tid].n);
        L.seg_S[tid] = ld_coh(&sr[tid].S);
    }
    const bool nuc = p.nucleus != 0;
    unsigned long long e[kChunk];
    const unsigned long long* lb = p.list + static_cast<size_t>(r) * p.nseg * kList;
#pragma unroll
    for (int c = 0; c < kChunk; ++c)
        e[c] = (nuc && c < p.nseg) ? ld_coh(lb + static_cast<size_t>(c) * kList + tid) : 0ull;
    if (tid == kThreads - 1) {
        // independent loads: the drafted token, and its logit as stored by the
        // segment holding it (meaningful only for a valid token)
        const int x = (j >= 0) ? p.draft_tokens[xi] : -1;
        const float zv = ld_coh(p.zx + r);
        L.n = x;
        L.zx = (j >= 0 && x >= 0 && x < p.V && !p.greedy) ? zv : 0.0f;
    }
    __syncthreads();
    if (tid < 64) {
        // row max (first segment holding it: lowest ids), deepest complete bin
        const int lane = tid;
        float bv = (lane < p.nseg) ? L.seg_m[lane] : -INFINITY;
        int bs = (lane < p.nseg) ? lane : 0x7FFFFFFF;
        int lo = (lane < p.nseg) ? L.seg_cut[lane] : -0x40000000;
        const int otop = (p.nseg <= 16) ? 16 : 64;  // lanes holding segments
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            if (o >= otop) continue;  // uniform
            const float ov = __shfl_xor(bv, o, 64);
            const int os = __shfl_xor(bs, o, 64);
            const bool take = (ov > bv) | ((ov == bv) & (os < bs));
            bv = take ? ov : bv;
            bs = take ? os : bs;
            lo = max(lo, __shfl_xor(lo, o, 64));
        }
        if (lane == 0) {
            L.m = bv;
            L.argmax = (bs < p.nseg) ? L.seg_kb[bs] : 0;
            L.kb_top = bin_of(bv, p.bscale);
            L.kb_lo = lo;
        }
        if (!p.greedy) {
            // normaliser relative to the row max (lane 0 holds it), in the same
            // wave: no barrier between the two
            const float mrow = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bv)));
            const float ms = (lane < p.nseg) ? L.seg_m[lane] : -INFINITY;
            const double sc = (ms == -INFINITY) ? 0.0 : weight(ms, mrow, p.invT, L.tab);
            if (lane < p.nseg) L.sc[lane] = sc;
            const double S = wave_sum((lane < p.nseg) ? L.seg_S[lane] * sc : 0.0);
            if (lane == 0) L.S = S;
        }
    }
    for (int i = tid; i < kBins; i += kThreads) { L.cand.hm[i] = 0.0; L.cand.hcnt[i] = 0; }
    if (tid == 0) { L.zk = -INFINITY; L.fastk = 1; L.Sk = 0.0; }
    __syncthreads();
    const float m = L.m;
    const int x = L.n;
    const bool x_ok = (x >= 0 && x < p.V);

    RowRec rec;
    rec.m = m;
    rec.tau = -INFINITY;
    rec.argmax = L.argmax;
    rec.kept = 1;
    rec.wx = 0.0;
    rec.S = 0.0;
    rec.fast = 0;
    rec.pad = 0;

    if (!p.greedy) {
        // top-k first (the k largest logits and their ties), from the lists'
        // bin counts or by radix select over the row
        float zk = -INFINITY;
        int fastk = 1;
        if (nuc && p.top_k > 0) {
            if (p.nseg <= kChunk) {
                const int kb_top = L.kb_top;
#pragma unroll
                for (int c = 0; c < kChunk; ++c) {
                    const int o = kb_top - bin_of(entry_z(e[c]), p.bscale);
                    const bool in = static_cast<int>(c < p.nseg) &
                                    static_cast<int>(tid < L.seg_n[min(c, p.nseg - 1)]) &
                                    static_cast<int>(o < kBins);
                    if (in) atomicAdd(&L.cand.hcnt[o], 1);
                }
            }
            __syncthreads();
            topk_lists(p, e, L);
            if (!L.fastk) {
                radix_threshold(p, row, m, 0.0, p.top_k, -INFINITY, L);
                if (tid == 0) { L.zk = L.tau; L.Sk = L.kept; }
                __syncthreads();
            }
            zk = L.zk;
            fastk = L.fastk;
        }
        if (nuc && p.nseg <= kChunk && fastk) {
            // bin masses of the listed entries with z >= zk, relative to the
            // row max: exact for every bin at or above kb_lo, which all lists
            // hold in full.  Weights of a batch are computed unconditionally
            // (independent chains; unused slots are masked), then added.
            const int kb_top = L.kb_top;
#pragma unroll
            for (int c0 = 0; c0 < kChunk; c0 += 4) {
                if (c0 >= p.nseg) break;  // uniform
                double wv[4];
                int ov[4];
                bool in[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = c0 + u;
                    const float zc = entry_z(e[c]);
                    ov[u] = kb_top - bin_of(zc, p.bscale);
                    in[u] = static_cast<int>(c < p.nseg) &
                            static_cast<int>(tid < L.seg_n[min(c, p.nseg - 1)]) &
                            static_cast<int>(ov[u] < kBins) & static_cast<int>(zc >= zk);
                    wv[u] = weight(zc, m, p.invT, L.tab);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (in[u]) atomicAdd(&L.cand.hm[ov[u]], wv[u]);
            }
        }
        __syncthreads();
        if (nuc && p.top_k > 0 && fastk) {
            // mass of the top-k set: every kept entry is listed (its bin is
            // at or above kb_lo and within kBins of the top)
            if (tid < 64) {
                double v = 0.0;
#pragma unroll
                for (int i = 0; i < kBinsPerLane; ++i) v += L.cand.hm[kBinsPerLane * tid + i];
                v = wave_sum(v);
                if (tid == 0) L.Sk = v;
            }
            __syncthreads();
        }
        rec.S = L.S;
        if (nuc) {
            const double Sk = (p.top_k > 0) ? L.Sk : L.S;
            if (p.top_p < 1.0) {
                const double target = p.top_p * Sk;
                if (fastk) {
                    list_threshold(p, target, zk, e, L);
                } else {
                    if (tid == 0) L.fast = 0;
                    __syncthreads();
                }
                if (!L.fast) radix_threshold(p, row, m, target, 0, zk, L);
                rec.tau = L.tau;
                rec.S = L.kept;
                rec.fast = L.fast;
            } else {
                rec.tau = zk;
                rec.S = Sk;
                rec.fast = fastk;
            }
        }
    }
    if (tid == 0) {
        if (j >= 0) {
            if (!x_ok) {
                set_status(p.status, 1);
                rec.kept = 0;
            } else if (!p.greedy) {
                rec.kept = (L.zx >= rec.tau) ? 1 : 0;
                rec.wx = weight(L.zx, m, p.invT, L.tab);
            }
        }
        RowRec* dst = p.rows + r;
        st_coh(&dst->m, rec.m);
        st_coh(&dst->tau, rec.tau);
        st_coh(&dst->S, rec.S);
        st_coh(&dst->wx, rec.wx);
        st_coh(&dst->kept, rec.kept);
        st_coh(&dst->argmax, rec.argmax);
        st_coh(&dst->fast, rec.fast);
    }
}

// ---------------------------------------------------------------- sequence

// The stopping row's parameters a draw needs (target q', draft p').
struct DrawRows {
    float mq, tq, mp, tp;  // row maxima and nucleus thresholds
    double Sq, Sp;         // kept masses
};

__device__ __forceinline__ DrawRows draw_rows(const RowRec& rq, const RowRec& rp) {
    return DrawRows{rq.m, rq.tau, rp.m, rp.tau, rq.S, rp.S};
}

// Draw weights of one element of the stopping row: residual (q'-p')_+ and q'.
// Branch-free: the weights are computed unconditionally and selected.
// Draw weights of one element, each up to a positive factor common to the
// whole row (the inverse-CDF draw is invariant to it): q' ~ w_q, and the
// residual (q' - p')_+ = (w_q/S_q - w_p/S_p)_+ ~ (w_q*S_p - w_p*S_q)_+.
// Both exps are computed unconditionally, so the calls of an unrolled loop
// are independent chains.
__device__ __forceinline__ void pair_weights(const DrawRows& R, bool residual, float zq, float zpv,
                                             bool valid, double invT, const double* tab, double* d,
                                             double* q) {
    const double wq = weight(zq, R.mq, invT, tab);
    const double wp = weight(zpv, R.mp, invT, tab);
    const double qv = (valid & (zq >= R.tq)) ? wq : 0.0;
    const double pv = (valid & residual & (zpv >= R.tp)) ? wp : 0.0;
    *q = qv;
    const double dd = fma(qv, R.Sp, -(pv * R.Sq));
    *d = residual ? (dd > 0.0 ? dd : 0.0) : qv;
}

// The draw over per-thread runs of elements in id order (thread t's run
// precedes thread t+1's).  Given this thread's sums `ds` (residual) and `qs`
// (q'), finds the crossing run with two block scans and returns, in every
// thread, the drawn id; `rescan(run, target, useq, &hit, &last)` walks this
// thread's run from the prefix `run`.  The residual falls back to q' when it
// has no mass.
template <typename RS>
__device__ __forceinline__ int draw_runs(const AcceptParams& p, int b, bool residual, double ds,
                                         double qs, RS rescan, RowsLds& L) {
    const int tid = threadIdx.x;
    double dt, qt;
    const double dx = block_excl_scan(ds, L.sq.scan, &dt);
    const double qx = block_excl_scan(qs, L.sq.scan, &qt);
    const bool useq = residual && !(dt > 0.0);
    const double tot = useq ? qt : dt;
    const float u = L.us;
    if (tid == 0 && !(u >= 0.0f && u < 1.0f)) set_status(p.status, 2);
    const double target = static_cast<double>(u) * tot;
    const double run0 = useq ? qx : dx;
    const double mine = useq ? qs : ds;
    if (tid == 0) { L.tok = 0x7FFFFFFF; L.lastpos = -1; }
    __syncthreads();
    if (mine > 0.0) {
        atomicMax(&L.lastpos, tid);
        if (run0 <= target && target < run0 + mine) {
            int hit = 0x7FFFFFFF, last = -1;
            rescan(run0, target, useq, &hit, &last);
            if (hit != 0x7FFFFFFF) atomicMin(&L.tok, hit);
        }
    }
    __syncthreads();
    if (L.tok == 0x7FFFFFFF) {
        // rounding left the target past every prefix: the last positive id
        if (tid == L.lastpos) {
            int hit = 0x7FFFFFFF, last = -1;
            rescan(run0, INFINITY, useq, &hit, &last);
            L.tok = last >= 0 ? last : 0;
        }
        __syncthreads();
        if (L.tok == 0x7FFFFFFF) return 0;
    }
    return L.tok;
}

// Token drawn at position n of sequence b from the stopping row's lists.  The
// residual (q'-p')_+ and q' vanish outside the target nucleus, so only list
// entries with z >= tau_q take part.  Thread t takes the contiguous run of
// flat list slots [t*E, (t+1)*E) (E = segments): list slots in (segment,
// slot) order are in id order, so the runs are too, and slots that are empty
// or below tau_q weigh zero.  The draft logits are fetched at the members'
// ids, one block scan of the (residual, q') run sums finds the run that holds
// the crossing, and E lanes of the owning thread's wave scan it (its entries
// read from that thread's registers with lane reads).
__device__ __forceinline__ int draw_from_lists(const AcceptParams& p, int b, int q0, int K, int n,
                                               RowsLds& L) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int rq = q0 + n;
    const bool residual = n < K;
    const DrawRows R = draw_rows(L.sq.rr[n], residual ? L.sq.rr[K + 1 + n] : L.sq.rr[n]);
    const int E0 = p.nseg;  // <= kChunk
    const unsigned long long* lb = p.list + static_cast<size_t>(rq) * p.nseg * kList;
    // one round trip: list lengths and every slot of this thread's run
    if (tid < p.nseg) L.seg_n[tid] = ld_coh(&p.seg[static_cast<size_t>(rq) * p.nseg + tid].n);
    unsigned long long e[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) e[i] = (i < E0) ? ld_coh(lb + tid * E0 + i) : 0ull;
    __syncthreads();
    // second round trip (residual): the draft logits at the members' ids
    const void* drow = row_ptr(p, p.nt + q0 - b + (residual ? n : 0));
    bool mem[kChunk];
    float zpv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const int lin = tid * E0 + i;
        mem[i] = static_cast<int>(i < E0) &
                 static_cast<int>((lin % kList) < L.seg_n[min(lin / kList, kMaxSeg - 1)]) &
                 static_cast<int>(entry_z(e[i]) >= R.tq);
        zpv[i] = (residual & mem[i]) ? load1(drow, p.bf16, entry_id(e[i])) : 0.0f;
    }
    double ds = 0.0, qs = 0.0;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (i < E0) {  // uniform: no work for slots past the row's segments
            double d, q;
            pair_weights(R, residual, entry_z(e[i]), zpv[i], mem[i], p.invT, L.tab, &d, &q);
            ds += d;
            qs += q;
            L.sq.zpa[i * kThreads + tid] = zpv[i];
        }
    }
    double dt, qt;
    double dx, qx;
    if (tid == 0) { L.tok = 0x7FFFFFFF; L.lastpos = -1; }  // ordered by the scan's barriers
    block_excl_scan2(ds, qs, L.sq.scan, L.sq.scan2, &dx, &qx, &dt, &qt);
    const bool useq = residual && !(dt > 0.0);  // zero residual mass: fall back to q'
    const double tot = useq ? qt : dt;
    const float u = L.us;
    if (tid == 0 && !(u >= 0.0f && u < 1.0f)) set_status(p.status, 2);
    const double target = static_cast<double>(u) * tot;
    const double run0 = useq ? qx : dx;
    const double mine = useq ? qs : ds;
    // the last run with positive mass (one atomic per wave), and the run that
    // holds the crossing (one thread at most)
    const unsigned long long posm = __ballot(mine > 0.0);
    if (posm && lane == 63 - __clzll(posm)) atomicMax(&L.lastpos, tid);
    if ((mine > 0.0) & (run0 <= target) & (target < run0 + mine)) L.tok = tid;
    __syncthreads();
    const bool tgt = (L.tok != 0x7FFFFFFF);
    const int owner = tgt ? L.tok : L.lastpos;  // rounding: last positive run
    if (owner < 0) return 0;  // uniform: no mass at all
    if ((tid >> 6) == (owner >> 6)) {
        // the owner's wave scans its run: lane i takes entry i, read from the
        // owner lane's registers
        const int ol = __builtin_amdgcn_readfirstlane(owner & 63);
        unsigned mm = 0;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) mm |= mem[i] ? (1u << i) : 0u;
        mm = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(mm), ol));
        const long long rb = __double_as_longlong(run0);
        const unsigned rlo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(rb), ol));
        const unsigned rhi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(rb >> 32), ol));
        const double r0 = __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(rhi) << 32) | rlo));
        unsigned long long ei = 0ull;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(e[i]), ol));
            const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(e[i] >> 32), ol));
            if (lane == i) ei = (static_cast<unsigned long long>(hi) << 32) | lo;
        }
        const bool ok = lane < E0;
        const bool is_mem = ok && ((mm >> min(lane, 31)) & 1u);
        double d = 0.0, q = 0.0;
        pair_weights(R, residual, entry_z(ei), L.sq.zpa[min(lane, kChunk - 1) * kThreads + owner],
                     is_mem, p.invT, L.tab, &d, &q);
        const double w = useq ? q : d;
        const double run = r0 + wave_incl_scan(w, lane);
        const unsigned long long hit = __ballot((w > 0.0) & (target < run) & tgt);
        const unsigned long long posb = __ballot(w > 0.0);
        int src = -1;
        if (hit) src = __ffsll(hit) - 1;
        else if (posb) src = 63 - __clzll(posb);
        const int id = entry_id(ei);
        const int tok = (src >= 0) ? __shfl(id, src, 64) : 0;
        if (lane == 0) L.n = tok;
    }
    __syncthreads();
    return L.n;
}

// Token drawn at position n of sequence b by one pass over the whole stopping
// row (rows whose lists do not hold the nucleus): thread t owns the
// contiguous ids [t*per, (t+1)*per).
__device__ __forceinline__ int draw_full_row(const AcceptParams& p, int b, int q0, int K, int n,
                                             RowsLds& L) {
    const int tid = threadIdx.x;
    const bool residual = n < K;
    const DrawRows R = draw_rows(L.sq.rr[n], residual ? L.sq.rr[K + 1 + n] : L.sq.rr[n]);
    const void* qrow = row_ptr(p, q0 + n);
    const void* prow = residual ? row_ptr(p, p.nt + q0 - b + n) : qrow;
    const int per = (p.V + kThreads - 1) / kThreads;
    const int e0 = min(p.V, tid * per), e1 = min(p.V, e0 + per);
    const int bf16 = p.bf16;
    const double invT = p.invT;
    double ds = 0.0, qs = 0.0;
    for (int e = e0; e < e1; ++e) {
        double d, q;
        pair_weights(R, residual, load1(qrow, bf16, e), residual ? load1(prow, bf16, e) : 0.0f,
                     true, invT, L.tab, &d, &q);
        ds += d;
        qs += q;
    }
    auto rescan = [&](double run, double target, bool useq, int* hit, int* last) {
        for (int e = e0; e < e1; ++e) {
            double d, q;
            pair_weights(R, residual, load1(qrow, bf16, e), residual ? load1(prow, bf16, e) : 0.0f,
                         true, invT, L.tab, &d, &q);
            const double w = useq ? q : d;
            if (w > 0.0) {
                *last = e;
                run += w;
                if (*hit == 0x7FFFFFFF && target < run) *hit = e;
            }
        }
    };
    return draw_runs(p, b, residual, ds, qs, rescan, L);
}

// Accept scan of sequence b once all of its rows are final; with the nucleus
// on (or greedy) also the emitted token.
__device__ __forceinline__ void finalize_sequence(const AcceptParams& p, int b, RowsLds& L) {
    const int tid = threadIdx.x;
    const int q0 = seq_q0(p, b);  // uniform
    const int K = seq_kb(p, b);   // this sequence's draft length
    const int d0 = q0 - b;        // its first draft token / draft row
    const int nt = p.nt;
    const int nr = p.greedy ? K + 1 : 2 * K + 1;
    __syncthreads();  // the row merge's LDS use ends
    // one round trip: the sequence's row records, drafts and uniforms
    if (tid < nr) {
        const int r = (tid <= K) ? q0 + tid : nt + d0 + (tid - K - 1);
        const RowRec* src = p.rows + r;
        L.sq.rr[tid].m = ld_coh(&src->m);
        L.sq.rr[tid].tau = ld_coh(&src->tau);
        L.sq.rr[tid].S = ld_coh(&src->S);
        L.sq.rr[tid].wx = ld_coh(&src->wx);
        L.sq.rr[tid].kept = ld_coh(&src->kept);
        L.sq.rr[tid].argmax = ld_coh(&src->argmax);
        L.sq.rr[tid].fast = ld_coh(&src->fast);
    }
    if (tid >= 128 && tid - 128 < K) {
        L.sq.x[tid - 128] = p.draft_tokens[d0 + tid - 128];
        L.sq.ua[tid - 128] = p.greedy ? 0.0f : p.u_accept[d0 + tid - 128];
    }
    if (tid == kThreads - 1) L.us = p.greedy ? 0.0f : p.u_sample[b];
    __syncthreads();
    if (tid < 64) {
        // every position's test at once (lane jj); n = first rejection
        const int jj = tid;
        bool acc = true;
        if (jj < K) {
            const RowRec& tr = L.sq.rr[jj];
            if (p.greedy) {
                acc = (L.sq.x[jj] == tr.argmax);
            } else {
                const RowRec& dr = L.sq.rr[K + 1 + jj];
                const double q = tr.kept ? tr.wx / tr.S : 0.0;
                const double pp = dr.kept ? dr.wx / dr.S : 0.0;
                const float u = L.sq.ua[jj];
                if (!(u >= 0.0f && u < 1.0f)) set_status(p.status, 2);
                acc = (pp > 0.0) ? (static_cast<double>(u) * pp < q) : (q > 0.0);
            }
        }
        const unsigned long long rej = __ballot(jj < K && !acc);
        if (jj == 0) L.n = rej ? __ffsll(rej) - 1 : K;
    }
    __syncthreads();
    if (tid == 0) {
        const int n = L.n;
        int32_t* out = p.out_tokens + q0;
        for (int i = 0; i < n; ++i) out[i] = L.sq.x[i];
        for (int i = n + 1; i <= K; ++i) out[i] = -1;
        if (p.greedy) out[n] = L.sq.rr[n].argmax;
        p.n_accepted[b] = n;
        p.seqs[b].n = n;
    }
    __syncthreads();
    if (p.greedy || !p.nucleus) return;  // no nucleus: draw_kernel draws
    const int n = L.n;
    int tok = L.sq.rr[n].fast ? draw_from_lists(p, b, q0, K, n, L) : -1;
    if (tok < 0) tok = draw_full_row(p, b, q0, K, n, L);
    if (tid == 0) p.out_tokens[q0 + n] = tok;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void rows_kernel(AcceptParams p) {
    __shared__ RowsLds L;
    const int tid = threadIdx.x;
    const int total = p.grid_rows * p.nseg;
    const int logical = xcd_remap(blockIdx.x, total);
    const int r = logical / p.nseg, s = logical % p.nseg;
    if (r >= p.nrows) return;
    const void* row = row_ptr(p, r);

    const int nt = p.nt;
    if (tid == 0) L.rb = 0;
    float z[kPerThread];
    load_segment(row, p.bf16, p.vec, p.V, s, tid, z);
    fill_exp_table(L.tab);
    // sequence of row r (ragged: the one whose target or draft rows hold it)
    int br;
    if (p.cu_q) {
        const bool tgt = r < nt;
        const int key = tgt ? r : r - nt;
        __syncthreads();
        for (int i = tid; i < p.B; i += kThreads) {
            const int lo = p.cu_q[i] - (tgt ? 0 : i), hi = p.cu_q[i + 1] - (tgt ? 0 : i + 1);
            if ((key >= lo) & (key < hi)) L.rb = i;
        }
        __syncthreads();
        br = L.rb;
    } else {
        br = (r < nt) ? r / (p.K + 1) : (r - nt) / p.K;
    }
    // drafted token of this row (target row j < K_b: draft index r - b; draft
    // row: r - nt); the segment holding it stores its logit for the merge
    const int xi = (r < nt) ? ((r + 1 < seq_q0(p, br + 1)) ? r - br : -1) : r - nt;
    const int xr = ((!p.greedy) & (xi >= 0)) ? p.draft_tokens[xi] : -1;
    if ((xr >= s * kSeg) & (xr < (s + 1) * kSeg) & (xr < p.V)) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
            if (seg_index(s, tid, k) == xr) st_coh(p.zx + r, z[k]);
    }
    __syncthreads();

    if (p.greedy) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            int e = seg_index(s, tid, k);
            const bool take = (e < p.V) & ((z[k] > bv) | ((z[k] == bv) & (e < bi)));
            bv = take ? z[k] : bv;
            bi = take ? e : bi;
        }
        // (value desc, index asc) reduction
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
        __shared__ float gv[kThreads / 64];
        __shared__ int gi[kThreads / 64];
        if ((tid & 63) == 0) { gv[tid >> 6] = bv; gi[tid >> 6] = bi; }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kThreads / 64; ++w)
                if (gv[w] > bv || (gv[w] == bv && gi[w] < bi)) { bv = gv[w]; bi = gi[w]; }
            SegHead* dst = p.seg + static_cast<size_t>(r) * p.nseg + s;
            st_coh(&dst->m, bv);
            st_coh(&dst->kb_top, bi);
        }
    } else {
        float lm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) lm = fmaxf(lm, z[k]);
        const float ms = block_max<kThreads>(lm, L.red_f);
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
            acc += (ms == -INFINITY) ? 0.0 : weight(z[k], ms, p.invT, L.tab);
        const double Ss = block_sum<kThreads>(acc, L.red_d);
        if (p.nucleus) {
            segment_list(p, r, s, z, ms, Ss, L);
        } else if (tid == 0) {
            SegHead* dst = p.seg + static_cast<size_t>(r) * p.nseg + s;
            st_coh(&dst->m, ms);
            st_coh(&dst->kb_top, bin_of(ms, p.bscale));
            st_coh(&dst->S, Ss);
        }
    }

    if (!arrive_last(p.row_cnt + r, p.nseg, &L.flag)) return;
    // the merges are the critical path: their waves issue ahead of the
    // segment work still running on the same compute unit
    __builtin_amdgcn_s_setprio(3);
    finalize_row(p, r, br, L);

    const int b = br;
    const int kb = seq_kb(p, b);
    const int rows_per_seq = p.greedy ? kb + 1 : 2 * kb + 1;
    if (!arrive_last(p.seq_cnt + b, rows_per_seq, &L.flag)) return;
    finalize_sequence(p, b, L);
}

// ---------------------------------------------------------------- draw

struct DrawLds {
    double tab[64];
    double red_d[kThreads / 64];
    double red_d2[kThreads / 64];
    int flag;
    RowRec rr[2];
    int n;
    double ds[kMaxSeg];
    double qs[kMaxSeg];
    double scan[kThreads];
    int tok;
    int last_pos;
    int sstar;
    int useq;
    double C;
    double target;
};

// Draw weights of one element of the stopping row: residual (q'-p')_+ or q'.
struct DrawCtx {
    const double* tab;
    const void* qrow;
    const void* prow;
    RowRec rq, rp;
    double invSq, invSp;
    int residual;
};

__device__ __forceinline__ void draw_weights(const DrawCtx& c, const AcceptParams& p, float zq,
                                             float zp, bool valid, double* w, double* qv) {
    const double wq = weight(zq, c.rq.m, p.invT, c.tab) * c.invSq;
    const double q = (valid & (zq >= c.rq.tau)) ? wq : 0.0;
    *qv = q;
    if (c.residual) {
        const double wp = weight(zp, c.rp.m, p.invT, c.tab) * c.invSp;
        const double pv = (valid & (zp >= c.rp.tau)) ? wp : 0.0;
        const double d = q - pv;
        *w = d > 0.0 ? d : 0.0;
    } else {
        *w = q;
    }
}

__global__ __launch_bounds__(kThreads) void draw_kernel(AcceptParams p, int grid_seqs) {
    __shared__ DrawLds L;
    const int tid = threadIdx.x;
    const int total = grid_seqs * p.nseg;
    const int logical = xcd_remap(blockIdx.x, total);
    const int b = logical / p.nseg, s = logical % p.nseg;
    if (b >= p.B) return;
    const int K = seq_kb(p, b), q0 = seq_q0(p, b), nt = p.nt;

    if (tid == 0) L.n = min(max(p.seqs[b].n, 0), K);
    fill_exp_table(L.tab);
    __syncthreads();
    const int n = L.n;
    if (tid == 0) L.rr[0] = p.rows[q0 + n];
    if (tid == 1 && n < K) L.rr[1] = p.rows[nt + q0 - b + n];
    __syncthreads();

    DrawCtx c;
    c.tab = L.tab;
    c.residual = n < K;
    c.qrow = row_ptr(p, q0 + n);
    c.rq = L.rr[0];
    c.invSq = 1.0 / c.rq.S;
    if (c.residual) {
        c.prow = row_ptr(p, nt + q0 - b + n);
        c.rp = L.rr[1];
        c.invSp = 1.0 / c.rp.S;
    } else {
        c.prow = nullptr;
        c.rp = c.rq;
        c.invSp = 0.0;
    }

    float zq[kPerThread], zp[kPerThread];
    load_segment(c.qrow, p.bf16, p.vec, p.V, s, tid, zq);
    if (c.residual) load_segment(c.prow, p.bf16, p.vec, p.V, s, tid, zp);
    double ws = 0.0, qs = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        double w, qv;
        const bool valid = seg_index(s, tid, k) < p.V;
        draw_weights(c, p, zq[k], c.residual ? zp[k] : 0.0f, valid, &w, &qv);
        ws += w;
        qs += qv;
    }
    ws = block_sum<kThreads>(ws, L.red_d);
    qs = block_sum<kThreads>(qs, L.red_d2);
    if (tid == 0) {
        st_coh(p.dsum + static_cast<size_t>(b) * p.nseg + s, ws);
        st_coh(p.qsum + static_cast<size_t>(b) * p.nseg + s, qs);
    }
    if (!arrive_last(p.draw_cnt + b, p.nseg, &L.flag)) return;

    // ---- last segment of sequence b: every segment sum in one round trip
    if (tid < p.nseg) {
        L.ds[tid] = ld_coh(p.dsum + static_cast<size_t>(b) * p.nseg + tid);
        L.qs[tid] = ld_coh(p.qsum + static_cast<size_t>(b) * p.nseg + tid);
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int t = 0; t < p.nseg; ++t) tot += L.ds[t];
        int useq = 0;
        if (c.residual && !(tot > 0.0)) {  // zero residual mass: fall back to q'
            useq = 1;
            tot = 0.0;
            for (int t = 0; t < p.nseg; ++t) tot += L.qs[t];
        }
        const float u = p.u_sample[b];
        if (!(u >= 0.0f && u < 1.0f)) set_status(p.status, 2);
        const double target = static_cast<double>(u) * tot;
        const double* v = useq ? L.qs : L.ds;
        double C = 0.0, Clast = 0.0;
        int sstar = -1, lastpos = 0;
        for (int t = 0; t < p.nseg; ++t) {
            if (v[t] > 0.0) { lastpos = t; Clast = C; }
            if (target < C + v[t]) { sstar = t; break; }
            C += v[t];
        }
        if (sstar < 0) { sstar = lastpos; C = Clast; }
        L.sstar = sstar;
        L.C = C;
        L.target = target;
        L.useq = useq;
        L.tok = 0x7FFFFFFF;
        L.last_pos = -1;
    }
    __syncthreads();
    const int ss = L.sstar;
    const double target = L.target;
    // contiguous layout for the exact in-order scan: thread t owns 16 ids
    const int e0 = ss * kSeg + tid * kPerThread;
    float q4[16], p4[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        load4(c.qrow, p.bf16, p.vec, p.V, e0 + 4 * i, q4 + 4 * i);
        if (c.residual) load4(c.prow, p.bf16, p.vec, p.V, e0 + 4 * i, p4 + 4 * i);
    }
    double w[kPerThread];
    double loc = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        double ww, qv;
        const bool valid = e0 + k < p.V;
        draw_weights(c, p, q4[k], c.residual ? p4[k] : 0.0f, valid, &ww, &qv);
        w[k] = L.useq ? qv : ww;
        loc += w[k];
    }
    // exclusive scan of per-thread sums (thread order = id order)
    const int lane = tid & 63, wv = tid >> 6;
    const double inc = wave_incl_scan(loc, lane);
    L.scan[tid] = inc;
    __syncthreads();
    double off = L.C;
    for (int u = 0; u < wv; ++u) off += L.scan[u * 64 + 63];
    double run = off + inc - loc;
    int mine = 0x7FFFFFFF, lastpos = -1;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        if (w[k] > 0.0) lastpos = e0 + k;
        run += w[k];
        mine = ((mine == 0x7FFFFFFF) & (w[k] > 0.0) & (target < run)) ? e0 + k : mine;
    }
    // ids increase with the thread: the wave's smallest candidate is its first
    // lane's with one, its largest positive id its last lane's (one LDS
    // atomic per wave instead of one per thread)
    const unsigned long long hasm = __ballot(mine != 0x7FFFFFFF);
    const unsigned long long hasl = __ballot(lastpos >= 0);
    if (hasm && lane == __ffsll(hasm) - 1) atomicMin(&L.tok, mine);
    if (hasl && lane == 63 - __clzll(hasl)) atomicMax(&L.last_pos, lastpos);
    __syncthreads();
    if (tid == 0) {
        int tok = L.tok != 0x7FFFFFFF ? L.tok : L.last_pos;
        if (tok < 0) tok = 0;
        p.out_tokens[q0 + n] = tok;
    }
}

}  // namespace

size_t accept_workspace_bytes(int B, long long nt, int V) {
    const size_t nseg = (static_cast<size_t>(V) + kSeg - 1) / kSeg;
    const size_t nrows = static_cast<size_t>(2 * nt - B);  // target and draft rows
    size_t off = 0;
    auto take = [&](size_t bytes) { off = (off + 255) & ~static_cast<size_t>(255); off += bytes; };
    // arrival counters first, sized for any draft lengths of B sequences
    take(static_cast<size_t>(B) * sizeof(int));
    take(static_cast<size_t>(B) * sizeof(int));
    take(static_cast<size_t>(B) * kMaxRowsPerSeq * sizeof(int));
    take(nrows * nseg * sizeof(SegHead));
    take(nrows * nseg * kList * sizeof(unsigned long long));
    take(nrows * sizeof(RowRec));
    take(nrows * sizeof(float));
    take(static_cast<size_t>(B) * sizeof(SeqRec));
    take(static_cast<size_t>(B) * nseg * sizeof(double));
    take(static_cast<size_t>(B) * nseg * sizeof(double));
    return (off + 255) & ~static_cast<size_t>(255);
}

int accept_max_vocab() { return kMaxSeg * kSeg; }
int accept_max_drafts() { return 64; }

hipError_t accept_launch(const AcceptArgs& a, hipStream_t stream) {
    AcceptParams p{};
    p.target = a.target_logits;
    p.draft = a.draft_logits;
    p.draft_tokens = a.draft_tokens;
    p.u_accept = a.u_accept;
    p.u_sample = a.u_sample;
    p.n_accepted = a.n_accepted;
    p.out_tokens = a.out_tokens;
    p.status = a.status;
    p.B = a.B;
    p.K = a.K;
    p.cu_q = a.cu_q;
    p.nt = a.nt;
    p.V = a.V;
    p.nseg = (a.V + kSeg - 1) / kSeg;
    p.bf16 = a.bf16;
    p.vec = (a.V % 4 == 0) ? 1 : 0;
    p.greedy = a.greedy;
    p.top_k = (a.top_k > 0 && a.top_k < a.V) ? a.top_k : 0;
    p.nucleus = (!a.greedy && (a.top_p < 1.0f || p.top_k > 0)) ? 1 : 0;
    p.invT = 1.0 / static_cast<double>(a.temperature);
    p.top_p = static_cast<double>(a.top_p);
    p.bscale = static_cast<float>(16.0 / static_cast<double>(a.temperature));
    p.bscale_c = static_cast<float>(4.0 / static_cast<double>(a.temperature));
    p.nrows = a.greedy ? a.nt : 2 * a.nt - a.B;
    p.grid_rows = (p.nrows + 7) / 8 * 8;

    const size_t nseg = p.nseg;
    const size_t nrows_max = static_cast<size_t>(2 * a.nt - a.B);
    char* base = static_cast<char*>(a.workspace);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        off = (off + 255) & ~static_cast<size_t>(255);
        char* ptr = base + off;
        off += bytes;
        return ptr;
    };
    // arrival counters first: their place depends on B only (the rows of B
    // sequences are at most B * kMaxRowsPerSeq), so calls with other draft
    // lengths or vocabularies never put data over them
    p.seq_cnt = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * sizeof(int)));
    p.draw_cnt = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * sizeof(int)));
    p.row_cnt = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * kMaxRowsPerSeq * sizeof(int)));
    p.seg = reinterpret_cast<SegHead*>(take(nrows_max * nseg * sizeof(SegHead)));
    p.list = reinterpret_cast<unsigned long long*>(take(nrows_max * nseg * kList * sizeof(unsigned long long)));
    p.rows = reinterpret_cast<RowRec*>(take(nrows_max * sizeof(RowRec)));
    p.zx = reinterpret_cast<float*>(take(nrows_max * sizeof(float)));
    p.seqs = reinterpret_cast<SeqRec*>(take(static_cast<size_t>(a.B) * sizeof(SeqRec)));
    p.dsum = reinterpret_cast<double*>(take(static_cast<size_t>(a.B) * nseg * sizeof(double)));
    p.qsum = reinterpret_cast<double*>(take(static_cast<size_t>(a.B) * nseg * sizeof(double)));

    hipLaunchKernelGGL(rows_kernel, dim3(p.grid_rows * p.nseg), dim3(kThreads), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.greedy || p.nucleus) return err;
    const int grid_seqs = (a.B + 7) / 8 * 8;
    hipLaunchKernelGGL(draw_kernel, dim3(grid_seqs * p.nseg), dim3(kThreads), 0, stream, p,
                       grid_seqs);
    return hipGetLastError();
}

}  // namespace sv
