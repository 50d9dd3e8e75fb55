// Modified rejection sampling for a batch of verify rounds on gfx950.
//
// Method: "Accelerating Large Language Model Decoding with Speculative
// Sampling", section "Modified rejection sampling" and Theorem 1: accept draft
// x_j with probability min(1, q(x_j)/p(x_j)) left to right, resample the first
// rejected position from (q - p)_+, draw a bonus token from the last target
// row when all K drafts pass; temperature and the top-k / nucleus filters
// modify q and p first.
//
// verify_kernel<EPT>  grid = units x segments of 256*EPT logits.  A unit is a
//   target row r of sequence b at position j: for j < K_b it pairs with draft
//   row j of b (the drafted token x_j is tested on the pair), for j = K_b it
//   is the bonus row.
//   segment_kernel (256 threads per unit segment)
//            one workgroup reads the same segment (the same token ids) of
//            the unit's target and draft rows: per row the max, the fp64
//            mass relative to it and, with a filter on, the candidate list
//            (every element of the highest quarter-unit bins of z/T that fit
//            in the list, in id order; target entries also carry the draft
//            logit of their id) and the fp64 mass and count of each listed
//            bin.  A nucleus keeps the upper part of the distribution, so
//            the lists normally hold it whole.
//   merge_kernel (1024 threads per unit; after the segment kernel)
//            merges both rows of the unit at once, one half of the
//            workgroup per row: max, normaliser, the exact tie-closed
//            filter threshold (bin masses summed over the segments, then the
//            boundary bin's listed entries ranked), the accept test of x_j
//            and -- only after a rejection, or for the bonus row -- the drawn
//            token: (q' - p')_+ and q' vanish outside the target's kept set,
//            and every target list entry carries its draft logit, so the draw
//            walks the target lists in id order with no further load.  A row
//            whose lists do not hold its kept set falls back to a radix
//            select and a draw over the whole row.
//            The units of a sequence then count themselves in one 64-bit
//            word that also gathers one rejection bit per position; the last
//            one stops at the first rejection and writes the emitted tokens.
//   Two launches instead of a last-arriver hand-off inside one: the merges
//   are chains of dependent steps, and a workgroup of their own (16 waves,
//   eight per row, coalesced list loads) runs them several times faster than
//   the last segment workgroup could, while the segment kernel keeps the
//   registers and occupancy of a streaming pass.
// draw_kernel  (no filter) grid = sequences x segments: the draw needs every
//   token of the stopping row, so it runs after the units: fp64 residual or
//   bonus weights per segment; the last segment picks the crossing segment
//   and scans it exactly.
// Every quantity that decides a token is fp64; the exp of the logits is the
// table-driven fp64 exp of sv_math.h (table of 2^(j/256) built per workgroup).
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_math.h"

namespace sv {
namespace {

constexpr int kThreads = 256;        // segment kernel workgroup
constexpr int kMThreads = 1024;      // merge kernel workgroup: one unit, two rows
constexpr int kHalf = kMThreads / 2; // threads per row in a unit merge
constexpr int kRW = kHalf / 64;      // waves per row
constexpr int kQB = 64;              // quarter-unit bins of z/T below a top bin (16 units)
constexpr int kSlots = 8;            // list slots per merging thread (list path: nseg*klist <= 4096)
constexpr int kCap = 512;            // boundary-bin entries ranked per row
constexpr int kSub = 64;             // sub-bins of a boundary quarter bin (1/256 unit of z/T each)
constexpr int kListSegMax = 21;      // segments the list path merges (3072-logit segments)
constexpr int kMaxSeg = 88;          // V <= 262144 with 3072-logit segments
constexpr int kMaxDrafts = 64;
constexpr int kMaskBits = 56;        // rejection bits in the sequence arrival word
constexpr int kListCap = 256;        // list capacity of a segment (16 * EPT)
constexpr unsigned long long kArrive = 1ull << kMaskBits;

struct SegHead {
    float m;      // segment max (greedy: max value)
    int top;      // quarter bin floor(m * 4/T) (greedy: lowest index of the max)
    int ocut;     // quarter bins top .. top - ocut are listed completely (-1: none)
    int n;        // list length
    double S;     // fp64 sum of exp((z - m)/T) over the segment
};

struct RowRec {
    float m;      // row max
    float tau;    // filter threshold logit (-inf: no filter)
    double S;     // kept mass relative to m (the full normaliser without filter)
    double wx;    // exp((z[x] - m)/T) for the drafted token x of the unit
    int kept;     // drafted token inside the kept set
    int argmax;   // lowest id of the row maximum (greedy)
    int fast;     // the row's lists hold its kept set
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
    SegHead* seg;              // [nrows][nseg]
    unsigned long long* list;  // [nrows][nseg][klist]: (id << 32) | bits of z, ids ascending
    float* lzp;                // [nt][nseg][klist]: draft logit at each target entry's id
    double* bmass;             // [nrows][nseg][kQB]: mass of listed quarter bin top - o (rel. to the segment max)
    int* bcnt;                 // [nrows][nseg][kQB]: its element count
    RowRec* rows;              // [nrows]
    float* zx;                 // [nrows]: logit of the unit's drafted token
    int* utok;                 // [nt]: token drawn by a unit (after a rejection, or the bonus)
    SeqRec* seqs;              // [B]
    double* dsum;              // [B][nseg] draw_kernel segment sums
    double* qsum;
    unsigned long long* seq_word;  // [B]: arrivals (top bits) and rejection bits
    unsigned long long* seq_mask;  // [B]: rejection bits of sequences with K_b > kMaskBits
    int* draw_cnt;             // [B]
    // compaction fused into the call (spec_accept_compact; compact = 0: off)
    int32_t* kv_len;           // [B] in/out
    const int64_t* kv_start;   // [B]
    char* k_cache;             // [rows][row_bytes] in/out
    char* v_cache;
    const char* k_new;         // [nt][row_bytes]
    const char* v_new;
    int32_t* tokens_packed;    // [nt]
    int32_t* cu_tokens;        // [B+1]
    int* cmp_e;                // [B] workspace: tokens emitted per sequence
    int* cmp_cnt;              // workspace: sequences compacted so far (zero between calls)
    long long row_bytes;       // one KV row (Hkv * D * element size)
    int compact;
    // row statistics from the LM head (spec_accept_prestats): per row, parts
    // of its ids with their max and fp64 sum relative to it; [0] target rows
    // [nt][pre_parts], [1] draft rows; used by stochastic rows without a filter
    const float* pre_m[2];
    const double* pre_s[2];
    int pre_parts;
    int prestats;
    const int32_t* cu_q;       // [B+1] ragged draft lengths: target rows of b start at cu_q[b]
    int nt;                    // target rows (cu_q[B], or B*(K+1)); draft row d is row nt + d
    int B, K, V, nseg, klist, grid_units;
    int bf16, vec, filter, greedy;  // filter: top_p < 1 or top-k on
    int top_k;                 // keep the k largest logits and their ties (0: off)
    double yscale;             // 256 / (T ln 2): exp((z - m)/T) = 2^((z - m) * yscale / 256)
    double top_p;
    float qscale;              // 4 / T: the quarter bin of z is floor(z * qscale)
};

// Sequence b owns target rows q0 .. q0+K_b (q0 = cu_q[b], or b*(K+1)) and
// draft rows nt+q0-b .. nt+q0-b+K_b-1; its drafts and accept uniforms start at
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

// Segment element k of thread tid (segments of 256*EPT logits): id
// s*256*EPT + (k/4)*1024 + tid*4 + k%4.
template <int EPT>
__device__ __forceinline__ int seg_index(int s, int tid, int k) {
    return s * (kThreads * EPT) + (k >> 2) * 1024 + tid * 4 + (k & 3);
}

template <int EPT>
__device__ __forceinline__ void load_segment(const void* row, int bf16, int vec, int V, int s,
                                             int tid, float* z) {
    const int e0 = s * (kThreads * EPT);
    if (vec && e0 + kThreads * EPT <= V) {  // uniform: the whole segment lies in the row
        if (bf16) {
            const uint2* r2 = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + e0) + tid;
            uint2 w[EPT / 4];
#pragma unroll
            for (int g = 0; g < EPT / 4; ++g) w[g] = r2[g * kThreads];
#pragma unroll
            for (int g = 0; g < EPT / 4; ++g) {
                z[4 * g + 0] = __uint_as_float(w[g].x << 16);
                z[4 * g + 1] = __uint_as_float(w[g].x & 0xFFFF0000u);
                z[4 * g + 2] = __uint_as_float(w[g].y << 16);
                z[4 * g + 3] = __uint_as_float(w[g].y & 0xFFFF0000u);
            }
        } else {
            const float4* r4 = reinterpret_cast<const float4*>(static_cast<const float*>(row) + e0) + tid;
            float4 w[EPT / 4];
#pragma unroll
            for (int g = 0; g < EPT / 4; ++g) w[g] = r4[g * kThreads];
#pragma unroll
            for (int g = 0; g < EPT / 4; ++g) {
                z[4 * g + 0] = w[g].x;
                z[4 * g + 1] = w[g].y;
                z[4 * g + 2] = w[g].z;
                z[4 * g + 3] = w[g].w;
            }
        }
        return;
    }
#pragma unroll
    for (int g = 0; g < EPT / 4; ++g)
        load4(row, bf16, vec, V, e0 + g * 1024 + tid * 4, z + 4 * g);
}

__device__ __forceinline__ const void* row_ptr(const AcceptParams& p, int r) {
    const size_t es = p.bf16 ? 2 : 4;
    if (r < p.nt) return static_cast<const char*>(p.target) + static_cast<size_t>(r) * p.V * es;
    return static_cast<const char*>(p.draft) + static_cast<size_t>(r - p.nt) * p.V * es;
}

// Quarter-unit bin of z/T: floor(z * 4/T), the product clamped far outside
// any logit range (one med3) and floored and converted by one instruction.
__device__ __forceinline__ int qbin(float z, float qscale) {
    const float y = __builtin_amdgcn_fmed3f(z * qscale, -1.0e9f, 1.0e9f);
    int b;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(b) : "v"(y));
    return b;
}

// fp64 weight exp((z - m)/T) of logit z relative to the max m (z - m exact in
// double; ys = 256 / (T ln 2)).
__device__ __forceinline__ double weight(float z, float m, double ys, const double* tab) {
    return exp2_256((static_cast<double>(z) - static_cast<double>(m)) * ys, tab);
}

// Fill the 256-entry table 2^(j/256) of exp2_256 (workgroups of at least 256
// threads); the caller synchronises before use.
__device__ __forceinline__ void fill_exp_table(double* tab) {
    if (threadIdx.x < 256) tab[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) * (1.0 / 256.0));
}

// Order-preserving 32-bit key of a float (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t fkey(float z) {
    uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float entry_z(unsigned long long e) {
    return __uint_as_float(static_cast<unsigned>(e));
}
__device__ __forceinline__ int entry_id(unsigned long long e) { return static_cast<int>(e >> 32); }

__device__ __forceinline__ double lane_read_d(double v, int src) {
    const long long bits = __double_as_longlong(v);
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(bits), src));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(bits >> 32), src));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// ---------------------------------------------------------------- LDS layout

struct SegLds {                     // segment kernel: rows 0 (target) and 1 (draft)
    double tab[256];                // 2^(j/256) for exp2_256
    float red_f[2][4];
    double red_d[2][4];
    int hc[2][4][kQB + 64];         // per-wave counts of quarter bins top - o (+ a dummy per lane)
    int fit[2];                     // bins top .. top - fit + 1 fit in the list
    unsigned long long wtot[2][4];  // per-wave packed list counts
    double hm[2][kQB];              // fp64 masses of the listed bins
    unsigned long long stage[2][kListCap];  // list entries in id order
    float stzp[kListCap];           // the draft logits of the target entries
    float gv[4];                    // greedy: per-wave max and its lowest index
    int gi[4];
};

struct RowPart {                    // one row of a unit merge
    float seg_m[kMaxSeg];
    int seg_top[kMaxSeg];
    int seg_ocut[kMaxSeg];
    int seg_n[kMaxSeg];
    double seg_S[kMaxSeg];
    double bm[kListSegMax][kQB];    // listed bin masses of every segment
    union {
        int bc[kListSegMax][kQB];   // their counts (top-k)
        struct {
            unsigned long long ck[kCap + 8];  // (z desc, id asc) order keys of the boundary bin
            float rz[kCap];                   // z in rank order
            double rw[kCap];                  // weight relative to the row max, in rank order
        } rk;
    };
    double part[kRW][kQB];          // per-wave partial bin masses
    int cpart[kRW][kQB];            // and counts
    double mass[kQB];               // row bin masses (bins top - o)
    double sbm[kSub];               // sub-bins of the boundary bin: masses,
    uint32_t sbk[2][kSub];          // and the smallest and largest order key of z
    int wcnt[kRW];
    float m;                        // row max
    int top;                        // its quarter bin
    int ocmax;                      // row bins top - o with o <= ocmax are listed in every segment
    double S;                       // normaliser relative to m
    float zx;                       // logit of the drafted token
    int fast;                       // the lists decided the kept set
    int og;                         // boundary bin (offset from top)
    double above;                   // mass of the bins above it
    int ccount;                     // ranked (gathered) entries
    int needsub;                    // the nucleus boundary is to be found in bin og
    float zmin;                     // only entries with z >= zmin take part (top-k floor)
    double target;                  // the nucleus mass to reach (from the row max)
    float zk;                       // top-k threshold logit (-inf: off)
    int abovec;                     // top-k: count above the boundary bin
    double Sk;                      // mass of the top-k set
    float tau;                      // kept set: z >= tau
    double kept;                    // its mass relative to m
};

struct MergeLds {
    double tab[256];
    union {
        RowPart r[2];
        struct {                       // draw: the kept target entries in id order
            float z[kHalf * kSlots];   // target logit
            float zp[kHalf * kSlots];  // draft logit at the same id
            int id[kHalf * kSlots];
        } dk;
    };
    struct {                        // radix select over a whole row
        double rh_m[256];
        int rh_c[256];
    } rad;
    double ta[kMThreads / 64];      // per-wave scan totals
    int dcnt[kSlots][kRW];          // draw: kept entries per (slot index, target wave)
    double tb[kMThreads / 64];
    uint32_t prefix, mask;
    int chosen, abovec;
    double above;
    float tau;
    double kept;
    int tok, lastpos, fstar;
    int seqn;                       // accepted drafts of the sequence (-1: not the last unit)
    int cflag;                      // compaction: this sequence arrived last
    int cscan[kMThreads / 64];      // compaction: per-wave scan totals
    int acc;                        // the unit's draft was accepted
    float us;                       // u_sample of the sequence
    float ua;                       // u_accept of the unit
};

// ---------------------------------------------------------------- segment pass

// Bin offset o = top - (quarter bin of z), capped at kQB (below the window).
__device__ __forceinline__ unsigned bin_off(float z, int top, float qscale) {
    return min(static_cast<unsigned>(top - qbin(z, qscale)), static_cast<unsigned>(kQB));
}

// Candidate lists of both rows of a unit segment (row 1 only if has_d), after
// the per-wave counts of the quarter bins top - o (o < kQB) are complete:
// the highest bins that fit in the list, the listed elements in id order
// ((id << 32) | bits of z; target entries also store the draft logit of
// their id), and the fp64 masses and counts of the listed bins.  ow holds the
// bin offsets of the thread's elements, four per word (kQB and above: below
// the window).  The elements are
// staged in LDS at their list positions, then stored with coalesced writes;
// the masses are taken over the staged entries, one per thread.
template <int EPT>
__device__ __forceinline__ void segment_lists(const AcceptParams& p, int s, int row0, int row1, bool has_d,
                                              const float (&z)[2][EPT], const unsigned (&ow)[2][EPT / 4],
                                              const int (&top)[2], const float* ms, SegLds& L) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nr = has_d ? 2 : 1;
    if (tid < 64 * nr) {
        // cumulative counts from the top bin down: bins 0 .. fit-1 fit (the
        // counts are nondecreasing in o)
        const int r = tid >> 6;
        const int rowr = r ? row1 : row0;
        const int c = (L.hc[r][0][lane] + L.hc[r][1][lane]) + (L.hc[r][2][lane] + L.hc[r][3][lane]);
        const int cum = wave_incl_scan(c, lane);
        const unsigned long long bal = __ballot(cum <= p.klist);
        if (lane == 0) L.fit[r] = __popcll(bal);
        if (p.top_k > 0) p.bcnt[(static_cast<size_t>(rowr) * p.nseg + s) * kQB + lane] = c;
    }
    __syncthreads();
    int ocut[2];
    unsigned long long packed[2] = {0ull, 0ull};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        ocut[r] = (r < nr) ? L.fit[r] - 1 : -1;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int o = static_cast<int>((ow[r][k >> 2] >> (8 * (k & 3))) & 0xFFu);
            packed[r] += (o <= ocut[r]) ? (1ull << (16 * (k >> 2))) : 0ull;
        }
    }
    // list positions in id order: 64-bit words of four 16-bit counters (one
    // per 1024-id group); no carry crosses a field
    unsigned long long inc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        inc[r] = wave_incl_scan(packed[r], lane);
        if (lane == 63) L.wtot[r][wv] = inc[r];
    }
    __syncthreads();
    int nlist[2] = {0, 0};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r >= nr) continue;  // uniform
        unsigned long long off = 0, tot = 0;
#pragma unroll
        for (int u = 0; u < kThreads / 64; ++u) {
            if (u < wv) off += L.wtot[r][u];
            tot += L.wtot[r][u];
        }
        const unsigned long long excl = off + inc[r] - packed[r];
        int gofs[EPT / 4];
        int run = 0;
#pragma unroll
        for (int g = 0; g < EPT / 4; ++g) {
            gofs[g] = run + static_cast<int>((excl >> (16 * g)) & 0xFFFF);
            run += static_cast<int>((tot >> (16 * g)) & 0xFFFF);
        }
        nlist[r] = run;
        const unsigned id0 = static_cast<unsigned>(seg_index<EPT>(s, tid, 0));
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int o = static_cast<int>((ow[r][k >> 2] >> (8 * (k & 3))) & 0xFFu);
            const int g = k >> 2;
            if (o <= ocut[r]) {
                const unsigned id = id0 + static_cast<unsigned>((k >> 2) * 1024 + (k & 3));
                L.stage[r][gofs[g]] = (static_cast<unsigned long long>(id) << 32) | __float_as_uint(z[r][k]);
                if (r == 0) L.stzp[gofs[g]] = z[1][k];
                ++gofs[g];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r >= nr) continue;  // uniform
        const size_t lbase = (static_cast<size_t>(r ? row1 : row0) * p.nseg + s) * p.klist;
        for (int t = tid; t < nlist[r]; t += kThreads) {
            const unsigned long long en = L.stage[r][t];
            p.list[lbase + t] = en;
            if (r == 0 && has_d) p.lzp[lbase + t] = L.stzp[t];
            const float ze = entry_z(en);
            atomicAdd(&L.hm[r][bin_off(ze, top[r], p.qscale)], weight(ze, ms[r], p.yscale, L.tab));
        }
    }
    __syncthreads();
    if (tid < 64 * nr) {
        // the listed bins only (the merge reads no bin below a segment's cut)
        const int r = tid >> 6;
        const int oc = r ? ocut[1] : ocut[0];
        if (lane <= oc) p.bmass[(static_cast<size_t>(r ? row1 : row0) * p.nseg + s) * kQB + lane] = L.hm[r][lane];
    }
    if (tid < nr) {
        const int r = tid;
        SegHead* h = p.seg + static_cast<size_t>(r ? row1 : row0) * p.nseg + s;
        h->m = r ? ms[1] : ms[0];
        h->top = r ? top[1] : top[0];
        h->ocut = r ? ocut[1] : ocut[0];
        h->n = r ? nlist[1] : nlist[0];
    }
}

// ---------------------------------------------------------------- radix select

// Exact tie-closed threshold of one row by radix select over the whole row
// (4 passes of 8 bits over order-preserving keys, fp64 digit masses and digit
// counts), among the elements with z >= zmin.  kcount > 0: the kcount-th
// largest value (top-k); else the filter boundary, the largest value whose
// tie-closed top set reaches `target` mass.  Sets L.tau and L.kept (mass of
// z >= tau, z >= zmin, relative to m).  All threads of the merge call it; the
// row arrives by value (an out-of-line call must not take the address of the
// kernel arguments).
struct RadixRow {
    const void* row;
    int V, bf16, vec;
    double ys;
};

__device__ __noinline__ void radix_threshold(RadixRow p, float m, double target, int kcount, float zmin,
                                             MergeLds& L) {
    const void* row = p.row;
    const int tid = threadIdx.x;
    if (tid == 0) { L.prefix = 0; L.mask = 0; L.above = 0.0; L.abovec = 0; }
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int d = tid; d < 256; d += kMThreads) { L.rad.rh_m[d] = 0.0; L.rad.rh_c[d] = 0; }
        __syncthreads();
        const uint32_t prefix = L.prefix, mask = L.mask;
        for (int base = 0; base < p.V; base += kMThreads * 16) {
            float z[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) load4(row, p.bf16, p.vec, p.V, base + (i * kMThreads + tid) * 4, z + 4 * i);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int e = base + ((k >> 2) * kMThreads + tid) * 4 + (k & 3);
                const uint32_t key = fkey(z[k]);
                if (e < p.V && (key & mask) == prefix && z[k] >= zmin) {
                    const int d = (key >> shift) & 0xFF;
                    atomicAdd(&L.rad.rh_m[d], weight(z[k], m, p.ys, L.tab));
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

// ---------------------------------------------------------------- unit merge

// Int wave minimum with DPP row shifts and broadcasts (every lane gets it).
__device__ __forceinline__ int wave_min_i(int v) {
    const int big = 0x7FFFFFFF;
    int r = min(v, dpp_i<0x111, 0xF, 0xF>(v, big));
    r = min(r, dpp_i<0x112, 0xF, 0xF>(v, big));
    r = min(r, dpp_i<0x113, 0xF, 0xF>(v, big));
    r = min(r, dpp_i<0x114, 0xF, 0xE>(r, big));
    r = min(r, dpp_i<0x118, 0xF, 0xC>(r, big));
    r = min(r, dpp_i<0x142, 0xA, 0xF>(r, big));
    r = min(r, dpp_i<0x143, 0xC, 0xF>(r, big));
    return __builtin_amdgcn_readlane(r, 63);
}

// Segment and slot of flat list slot f (klist is 192 or 256).
__device__ __forceinline__ void slot_pos(int f, int klist, int* sg, int* o) {
    const int s = (klist == 256) ? (f >> 8) : ((f >> 6) / 3);
    *sg = s;
    *o = f - s * klist;
}

// Gather the listed entries of quarter bin R.top - R.og with z >= R.zmin from
// the slots of each row whose list path is on (want), and rank them by
// (z desc, id asc): R.rk.rz[rank] = z, R.rk.rw[rank] = fp64 weight relative to
// the row max, R.ccount = their number.  Clears R.fast when there are none or
// more than kCap.  All threads call it; each half works on its row (slot i of
// this thread is valid iff bit i of vmask).
__device__ __forceinline__ void rank_bin(const AcceptParams& p, const unsigned long long (&e)[kSlots],
                                         unsigned vmask, bool want, MergeLds& L) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int rr = tid / kHalf, rt = tid & (kHalf - 1), rw = rt >> 6;
    RowPart& R = L.r[rr];
    const bool go = want && R.fast;
    const int sel = R.top - R.og;
    const float zmin = R.zmin;
    unsigned long long bal[kSlots];
    int wcount = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const float zi = entry_z(e[i]);
        const bool in = go && ((vmask >> i) & 1u) && qbin(zi, p.qscale) == sel && zi >= zmin;
        bal[i] = __ballot(in);
        wcount += __popcll(bal[i]);
    }
    if (lane == 0) R.wcnt[rw] = wcount;
    __syncthreads();
    int base = 0, n = 0;
#pragma unroll
    for (int w2 = 0; w2 < kRW; ++w2) {
        const int c = R.wcnt[w2];
        base += (w2 < rw) ? c : 0;
        n += c;
    }
    const bool ok = go && n > 0 && n <= kCap;
    if (ok) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const unsigned long long bc = bal[i];
            const int slot = base + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bc >> 32),
                                                              __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bc), 0));
            if ((bc >> lane) & 1ull) {
                const uint32_t id = static_cast<uint32_t>(entry_id(e[i]));
                R.rk.ck[slot] = (static_cast<unsigned long long>(fkey(entry_z(e[i]))) << 32) | (0xFFFFFFFFu - id);
            }
            base += __popcll(bc);
        }
        for (int i = n + rt; i < ((n + 7) & ~7); i += kHalf) R.rk.ck[i] = 0ull;  // pad: never larger
    }
    if (rt == 0 && go) {
        R.ccount = n;
        if (!ok) R.fast = 0;
    }
    __syncthreads();
    if (ok) {
        // rank = number of larger keys (keys are distinct): each thread ranks
        // entries rt and rt + kHalf in one pass over the keys, which the
        // row's threads read together (LDS broadcast), 8 per batch
        const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(R.rk.ck);
        const bool h0 = rt < n, h1 = rt + kHalf < n;
        const unsigned long long c0 = h0 ? R.rk.ck[rt] : ~0ull;
        const unsigned long long c1 = h1 ? R.rk.ck[rt + kHalf] : ~0ull;
        int r0 = 0, r1 = 0;
#pragma unroll 4
        for (int jj = 0; jj < n; jj += 8) {
            const ulonglong2 a0 = k2[jj / 2], a1 = k2[jj / 2 + 1], a2 = k2[jj / 2 + 2], a3 = k2[jj / 2 + 3];
            r0 += static_cast<int>(a0.x > c0) + static_cast<int>(a0.y > c0) + static_cast<int>(a1.x > c0) +
                  static_cast<int>(a1.y > c0) + static_cast<int>(a2.x > c0) + static_cast<int>(a2.y > c0) +
                  static_cast<int>(a3.x > c0) + static_cast<int>(a3.y > c0);
            r1 += static_cast<int>(a0.x > c1) + static_cast<int>(a0.y > c1) + static_cast<int>(a1.x > c1) +
                  static_cast<int>(a1.y > c1) + static_cast<int>(a2.x > c1) + static_cast<int>(a2.y > c1) +
                  static_cast<int>(a3.x > c1) + static_cast<int>(a3.y > c1);
        }
        if (h0) {
            const float zi = fkey_inv(static_cast<uint32_t>(c0 >> 32));
            R.rk.rz[r0] = zi;
            R.rk.rw[r0] = weight(zi, R.m, p.yscale, L.tab);
        }
        if (h1) {
            const float zi = fkey_inv(static_cast<uint32_t>(c1 >> 32));
            R.rk.rz[r1] = zi;
            R.rk.rw[r1] = weight(zi, R.m, p.yscale, L.tab);
        }
    }
    __syncthreads();
}

// Sub-bin of z inside its quarter bin sel: 64 equal parts of the bin's width,
// in increasing z (y is the clamped z * 4/T of qbin; y - sel is exact below
// 2^24 and 0 above, where every z of a bin is one value).
__device__ __forceinline__ int sub_bin(float y, int sel) {
    return min(static_cast<int>((y - static_cast<float>(sel)) * static_cast<float>(kSub)), kSub - 1);
}

// Nucleus threshold inside quarter bin og of each row with R.needsub: the
// largest z whose tie-inclusive mass from the top (R.above, the bins above og,
// plus the entries of og with z >= that value and z >= R.zmin) reaches
// R.target; sets R.tau and R.kept.  The bin's listed entries are gathered
// (z, then their fp64 weights, one or two per thread) and spread over kSub
// sub-bins (mass, smallest and largest z); the first sub-bin from the top
// whose cumulative mass reaches the target holds the threshold.  When that
// sub-bin holds one value (bf16 logits nearly always), it is the threshold;
// otherwise each of its entries' tie-inclusive mass is summed exactly.  All
// threads call it; each half works on its row (slot i of this thread is valid
// iff bit i of vmask).  The sub-bin arrays start cleared.
__device__ __forceinline__ void subbin_threshold(const AcceptParams& p, const unsigned long long (&e)[kSlots],
                                                 unsigned vmask, MergeLds& L) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int rr = tid / kHalf, rt = tid & (kHalf - 1), rw = rt >> 6;
    RowPart& R = L.r[rr];
    const bool go = R.needsub != 0;
    const int sel = R.top - R.og;
    const float zfloor = R.zmin;
    // ---- gather the bin's entries
    unsigned long long bal[kSlots];
    int wcount = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const float zi = entry_z(e[i]);
        const bool in = go && ((vmask >> i) & 1u) && qbin(zi, p.qscale) == sel && zi >= zfloor;
        bal[i] = __ballot(in);
        wcount += __popcll(bal[i]);
    }
    if (lane == 0) R.wcnt[rw] = wcount;
    __syncthreads();
    int base = 0, n = 0;
#pragma unroll
    for (int w2 = 0; w2 < kRW; ++w2) {
        const int c = R.wcnt[w2];
        base += (w2 < rw) ? c : 0;
        n += c;
    }
    const bool ok = go && n <= kCap;
    if (ok) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const unsigned long long bc = bal[i];
            const int slot = base + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bc >> 32),
                                                              __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bc), 0));
            if ((bc >> lane) & 1ull) R.rk.rz[slot] = entry_z(e[i]);
            base += __popcll(bc);
        }
    }
    if (rt == 0 && go) {
        R.ccount = n;
        if (!ok) R.fast = 0;  // more than the gather holds: whole-row select
    }
    __syncthreads();
    // ---- weights and sub-bins
    if (ok) {
        for (int t = rt; t < n; t += kHalf) {
            const float zi = R.rk.rz[t];
            const float y = __builtin_amdgcn_fmed3f(zi * p.qscale, -1.0e9f, 1.0e9f);
            const int sb = sub_bin(y, sel);
            const uint32_t k = fkey(zi);
            const double w = weight(zi, R.m, p.yscale, L.tab);
            R.rk.rw[t] = w;
            atomicAdd(&R.sbm[sb], w);
            atomicMin(&R.sbk[0][sb], k);
            atomicMax(&R.sbk[1][sb], k);
        }
    }
    __syncthreads();
    if (ok && rw == 0) {
        const int sb = kSub - 1 - lane;  // lane 0: the highest sub-bin
        const double v = R.sbm[sb];
        const uint32_t kmin = R.sbk[0][sb], kmax = R.sbk[1][sb];
        const double target = R.target;
        const double cum = R.above + wave_incl_scan(v, lane);
        const unsigned long long hit = __ballot(kmax != 0u && cum >= target);
        const unsigned long long any = __ballot(kmax != 0u);
        // no sub-bin reaches the target (rounding between the bin and entry
        // sums): keep every entry, down to the lowest value
        const int star = hit ? __ffsll(hit) - 1 : (any ? 63 - __clzll(any) : 0);
        const double before = star > 0 ? __shfl(cum, star - 1, 64) : R.above;
        const double at = __shfl(cum, star, 64);
        const uint32_t smin = __shfl(kmin, star, 64), smax = __shfl(kmax, star, 64);
        if (!hit || smin == smax) {  // uniform: one value, or everything kept
            if (lane == 0) {
                R.tau = fkey_inv(smin);
                R.kept = at;
            }
        } else {
            // several values in the crossing sub-bin: this wave compacts its
            // entries (z and weight, in gather order) to the front of rz/rw
            // -- a slot is written only after the read of every slot up to
            // it -- and sums each one's tie-inclusive mass
            const int starsb = kSub - 1 - star;
            int m = 0;
            for (int c0 = 0; c0 < n; c0 += 256) {
                float zq[4];
                double wq[4];
#pragma unroll
                for (int h2 = 0; h2 < 4; ++h2) {  // the reads of four chunks at once (clamped ids)
                    const int i = min(c0 + 64 * h2 + lane, kCap - 1);
                    zq[h2] = R.rk.rz[i];
                    wq[h2] = R.rk.rw[i];
                }
#pragma unroll
                for (int h2 = 0; h2 < 4; ++h2) {
                    const int i = c0 + 64 * h2 + lane;
                    const bool in = i < n &&
                                    sub_bin(__builtin_amdgcn_fmed3f(zq[h2] * p.qscale, -1.0e9f, 1.0e9f), sel) ==
                                        starsb;
                    const unsigned long long bc = __ballot(in);
                    if (in) {
                        const int at2 = m + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bc >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bc), 0));
                        R.rk.rz[at2] = zq[h2];
                        R.rk.rw[at2] = wq[h2];
                    }
                    m += __popcll(bc);
                }
            }
            // the entries written by other lanes of this wave are read next
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // each lane's tie-inclusive mass sums the entries in gather order;
            // they are held 64 at a time in registers and broadcast lane by
            // lane (no LDS round trip per term)
            float best = -INFINITY, lowest = INFINITY;
            float zown = -INFINITY;  // this lane's entry when m <= 64
            double wown = 0.0;
            for (int c0 = 0; c0 < m; c0 += 64) {
                const int a2 = c0 + lane;
                const float zi = a2 < m ? R.rk.rz[a2] : INFINITY;
                double g = 0.0;
                for (int c1 = 0; c1 < m; c1 += 64) {
                    const int b2 = c1 + lane;
                    const float zb = b2 < m ? R.rk.rz[b2] : -INFINITY;
                    const double wb = b2 < m ? R.rk.rw[b2] : 0.0;
                    if (c0 == 0 && c1 == 0) {
                        zown = zb;
                        wown = wb;
                    }
                    const int nn = min(64, m - c1);
                    for (int jj = 0; jj < nn; ++jj) {
                        const float zj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zb), jj));
                        const double wj = lane_read_d(wb, jj);
                        g += (zj >= zi) ? wj : 0.0;
                    }
                }
                if (a2 < m) {
                    lowest = fminf(lowest, zi);
                    if (before + g >= target) best = fmaxf(best, zi);
                }
            }
            best = wave_max(best);
            lowest = -wave_max(-lowest);
            const float tau = (best != -INFINITY) ? best : lowest;
            double part = 0.0;
            if (m <= 64) {  // uniform
                part = (zown >= tau) ? wown : 0.0;
            } else {
                for (int c0 = 0; c0 < m; c0 += 64) {
                    const int a2 = c0 + lane;
                    if (a2 < m) part += (R.rk.rz[a2] >= tau) ? R.rk.rw[a2] : 0.0;
                }
            }
            part = wave_sum(part);
            if (lane == 0) {
                R.tau = tau;
                R.kept = before + part;
            }
        }
    }
    __syncthreads();
}

// The stopping row's parameters a draw needs (target q', draft p').
struct DrawRows {
    float mq, tq, mp, tp;  // row maxima and filter thresholds
    double Sq, Sp;         // kept masses
};

// Draw weights of one element, each up to a positive factor common to the
// whole row (the inverse-CDF draw is invariant to it): q' ~ w_q, and the
// residual (q' - p')_+ = (w_q/S_q - w_p/S_p)_+ ~ (w_q*S_p - w_p*S_q)_+.  Both
// exps are computed unconditionally, so the calls of an unrolled loop are
// independent chains.
__device__ __forceinline__ void pair_weights(const DrawRows& R, bool residual, float zq, float zpv,
                                             bool valid, double ys, const double* tab, double* d,
                                             double* q) {
    const double wq = weight(zq, R.mq, ys, tab);
    const double wp = weight(zpv, R.mp, ys, tab);
    const double qv = (valid & (zq >= R.tq)) ? wq : 0.0;
    const double pv = (valid & residual & (zpv >= R.tp)) ? wp : 0.0;
    *q = qv;
    const double dd = fma(qv, R.Sp, -(pv * R.Sq));
    *d = residual ? (dd > 0.0 ? dd : 0.0) : qv;
}

// Block-wide exclusive scan of one or two doubles per thread in thread order
// (fixed order); sa, sb hold the per-wave totals.
__device__ __forceinline__ void block_excl_scan2(double a, double b, double* sa, double* sb,
                                                 double* ea, double* eb, double* ta, double* tb) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const double ia = wave_incl_scan(a, lane);
    const double ib = wave_incl_scan(b, lane);
    __syncthreads();
    if (lane == 63) {
        sa[wv] = ia;
        sb[wv] = ib;
    }
    __syncthreads();
    double oa = 0.0, ob = 0.0, xa = 0.0, xb = 0.0;
#pragma unroll
    for (int u = 0; u < kMThreads / 64; ++u) {
        const double va = sa[u], vb = sb[u];
        if (u < wv) { oa += va; ob += vb; }
        xa += va;
        xb += vb;
    }
    *ta = xa;
    *tb = xb;
    *ea = oa + ia - a;
    *eb = ob + ib - b;
}

// The accept test's inputs: the unit's row records, read by one thread into
// registers (the draw reuses their LDS).
struct AcceptIn {
    float zq, mq, tq;   // target row: drafted logit, max, filter threshold
    float zp, mp, tp;   // draft row
    double Sq, Sp;      // kept masses relative to the maxima
    int fq, fp;         // the lists decided the kept sets
    float ua;           // u_accept of the unit
};

__device__ __forceinline__ AcceptIn accept_in(const MergeLds& L) {
    const RowPart& T = L.r[0];
    const RowPart& D = L.r[1];
    return AcceptIn{T.zx, T.m, T.tau, D.zx, D.m, D.tau, T.kept, D.kept, T.fast, D.fast, L.ua};
}

// The accept test of x_j (one thread): q'_j(x) = w_x / kept mass if x is
// kept, else 0; accept iff u * p' < q' (p' = 0: iff q' > 0).  Also stores
// the unit's row records.
__device__ __forceinline__ bool accept_decide(const AcceptParams& p, const AcceptIn& a, int u, int dr, int j,
                                              int kb, bool x_ok, const double* tab) {
    bool acc = true;
    const bool tk = x_ok && j < kb && a.zq >= a.tq;
    const double wxq = (x_ok && j < kb) ? weight(a.zq, a.mq, p.yscale, tab) : 0.0;
    RowRec* tr = p.rows + u;
    st_coh(&tr->m, a.mq);
    st_coh(&tr->tau, a.tq);
    st_coh(&tr->S, a.Sq);
    st_coh(&tr->wx, wxq);
    st_coh(&tr->kept, tk ? 1 : 0);
    st_coh(&tr->fast, a.fq);
    if (j < kb) {
        const bool dk = x_ok && a.zp >= a.tp;
        const double wxp = x_ok ? weight(a.zp, a.mp, p.yscale, tab) : 0.0;
        RowRec* drr = p.rows + dr;
        st_coh(&drr->m, a.mp);
        st_coh(&drr->tau, a.tp);
        st_coh(&drr->S, a.Sp);
        st_coh(&drr->wx, wxp);
        st_coh(&drr->kept, dk ? 1 : 0);
        st_coh(&drr->fast, a.fp);
        if (!x_ok) set_status(p.status, 1);
        const double q = tk ? wxq / a.Sq : 0.0;
        const double pp = dk ? wxp / a.Sp : 0.0;
        if (!(a.ua >= 0.0f && a.ua < 1.0f)) set_status(p.status, 2);
        acc = (pp > 0.0) ? (static_cast<double>(a.ua) * pp < q) : (q > 0.0);
    }
    return acc;
}

// The accept test on thread 0; every thread returns the decision.
__device__ __forceinline__ bool accept_test(const AcceptParams& p, int u, int dr, int j, int kb, bool x_ok,
                                            MergeLds& L) {
    if (threadIdx.x == 0) L.acc = accept_decide(p, accept_in(L), u, dr, j, kb, x_ok, L.tab) ? 1 : 0;
    __syncthreads();
    return L.acc != 0;
}

// Block-wide exclusive scan of one double per thread in thread order (fixed
// order); sa holds the per-wave totals.  The caller has passed a barrier since
// sa was last read.
__device__ __forceinline__ void block_excl_scan1(double a, double* sa, double* ea, double* ta) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const double ia = wave_incl_scan(a, lane);
    if (lane == 63) sa[wv] = ia;
    __syncthreads();
    double oa = 0.0, xa = 0.0;
#pragma unroll
    for (int u = 0; u < kMThreads / 64; ++u) {
        const double va = sa[u];
        if (u < wv) oa += va;
        xa += va;
    }
    *ta = xa;
    *ea = oa + ia - a;
}

// Token drawn by a unit from its target row's lists (every thread returns it;
// -1 when the residual has no mass).
// The target half's thread rt holds flat slots rt + kHalf*i (coalesced
// loads), so the order (i, wave, lane) is id order.  The kept entries (valid
// slots with z >= tau_q: q' and (q' - p')_+ vanish elsewhere) are compacted
// in that order with their draft logits; the whole workgroup then takes runs
// of consecutive entries, computes the draw weights -- (q' - p')_+, or q'
// for the bonus row -- sums and scans the runs, and the run holding the
// crossing is walked.  The accept test of the unit's draft runs inside, on
// the last thread (ai holds its inputs there), and leaves its decision in
// L.acc; the draw is made whatever the decision.
__device__ __forceinline__ int draw_from_lists(const AcceptParams& p, const DrawRows& R, bool residual,
                                               float us, const unsigned long long (&e)[kSlots],
                                               const float (&zpv)[kSlots], unsigned vmask, const AcceptIn& ai,
                                               int u, int dr, int j, int kb, bool x_ok, MergeLds& L) {
    static_assert(kHalf * kSlots <= 4 * kMThreads, "at most four kept entries per thread");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool tg = tid < kHalf;
    unsigned long long bal[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i)
        bal[i] = __ballot(tg && ((vmask >> i) & 1u) && entry_z(e[i]) >= R.tq);
    if (tg && lane == 0) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) L.dcnt[i][wv] = __popcll(bal[i]);
    }
    if (tid == 0) {
        L.fstar = 0x7FFFFFFF;
        L.lastpos = -1;
        if (!(us >= 0.0f && us < 1.0f)) set_status(p.status, 2);
    }
    // every thread holds its row parameters (R, ai) in registers: the kept
    // entries overwrite the row records (they share LDS)
    __syncthreads();
    // offsets of the kept entries: one wave scan over the counts in (slot
    // index, wave) order, each wave reads its own eight
    static_assert(kSlots * kRW == 64, "one count per lane");
    const int cnt = (&L.dcnt[0][0])[lane];
    const int inc = wave_incl_scan(cnt, lane);
    const int n = __builtin_amdgcn_readlane(inc, 63);
    const int exc = inc - cnt;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    int base[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) base[i] = __builtin_amdgcn_readlane(exc, i * kRW + (wvu & (kRW - 1)));
    if (tg) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const unsigned long long bc = bal[i];
            if ((bc >> lane) & 1ull) {
                const int c = base[i] + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bc >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bc), 0));
                L.dk.z[c] = entry_z(e[i]);
                L.dk.zp[c] = zpv[i];
                L.dk.id[c] = entry_id(e[i]);
            }
        }
    }
    __syncthreads();
    // runs of E consecutive kept entries (E <= 4), weights summed in id order
    const int E = (n + kMThreads - 1) / kMThreads;
    const int c0 = min(tid * E, n), c1 = min(c0 + E, n);
    double w[4];
    double mine = 0.0;
    int lastc = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = c0 + k;
        double d = 0.0, q;
        if (c < c1) pair_weights(R, residual, L.dk.z[c], L.dk.zp[c], true, p.yscale, L.tab, &d, &q);
        w[k] = d;
        mine += d;
        if (d > 0.0) lastc = c;
    }
    if (tid == kMThreads - 1) L.acc = accept_decide(p, ai, u, dr, j, kb, x_ok, L.tab) ? 1 : 0;
    double rx, tot;
    block_excl_scan1(mine, L.ta, &rx, &tot);
    // the residual has mass (it can lack it through rounding only: then the
    // caller draws from q' over the whole row)
    if (residual && !(tot > 0.0)) return -1;  // uniform
    const double target = static_cast<double>(us) * tot;
    if ((mine > 0.0) & (rx <= target) & (target < rx + mine)) {
        double run = rx;
        int hit = -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (hit < 0 && w[k] > 0.0) {
                run += w[k];
                if (target < run) hit = c0 + k;
            }
        }
        if (hit >= 0) L.fstar = hit;
    }
    // the last entry of positive weight (rounding left the target past every
    // prefix); entries grow with the thread, so one atomic per wave
    const unsigned long long hasl = __ballot(lastc >= 0);
    if (hasl && lane == 63 - __clzll(hasl)) atomicMax(&L.lastpos, lastc);
    __syncthreads();
    const int fs = (L.fstar != 0x7FFFFFFF) ? L.fstar : L.lastpos;
    if (fs < 0) return 0;  // uniform: no mass at all
    return L.dk.id[fs];
}

// Token drawn from the unit's target row by one pass over the whole row
// (rows whose lists do not hold the kept set, or rows beyond the list path):
// thread t owns the contiguous ids [t*per, (t+1)*per).
struct FullRow {
    const void* qrow;
    const void* prow;
    int32_t* status;
    int V, bf16;
    double ys;
};

__device__ __noinline__ int draw_full_row(FullRow p, DrawRows R, bool residual, float us, MergeLds& L) {
    const void* qrow = p.qrow;
    const void* prow = p.prow;
    const int tid = threadIdx.x;
    const int per = (p.V + kMThreads - 1) / kMThreads;
    const int e0 = min(p.V, tid * per), e1 = min(p.V, e0 + per);
    const int bf16 = p.bf16;
    const double ys = p.ys;
    double ds = 0.0, qs = 0.0;
    for (int e = e0; e < e1; ++e) {
        double d, q;
        pair_weights(R, residual, load1(qrow, bf16, e), residual ? load1(prow, bf16, e) : 0.0f, true,
                     ys, L.tab, &d, &q);
        ds += d;
        qs += q;
    }
    if (tid == 0) { L.tok = 0x7FFFFFFF; L.lastpos = -1; }
    double dx, qx, dt, qt;
    block_excl_scan2(ds, qs, L.ta, L.tb, &dx, &qx, &dt, &qt);
    const bool useq = residual && !(dt > 0.0);
    const double tot = useq ? qt : dt;
    if (tid == 0 && !(us >= 0.0f && us < 1.0f)) set_status(p.status, 2);
    const double target = static_cast<double>(us) * tot;
    const double mine = useq ? qs : ds;
    double run = useq ? qx : dx;
    if (mine > 0.0) {
        atomicMax(&L.lastpos, tid);
        if (run <= target && target < run + mine) {
            int hit = 0x7FFFFFFF;
            for (int e = e0; e < e1; ++e) {
                double d, q;
                pair_weights(R, residual, load1(qrow, bf16, e), residual ? load1(prow, bf16, e) : 0.0f,
                             true, ys, L.tab, &d, &q);
                const double w = useq ? q : d;
                if (w > 0.0) {
                    run += w;
                    if (hit == 0x7FFFFFFF && target < run) hit = e;
                }
            }
            if (hit != 0x7FFFFFFF) atomicMin(&L.tok, hit);
        }
    }
    __syncthreads();
    if (L.tok == 0x7FFFFFFF) {
        // rounding left the target past every prefix: the last positive id
        if (tid == L.lastpos) {
            int last = -1;
            for (int e = e0; e < e1; ++e) {
                double d, q;
                pair_weights(R, residual, load1(qrow, bf16, e), residual ? load1(prow, bf16, e) : 0.0f,
                             true, ys, L.tab, &d, &q);
                if ((useq ? q : d) > 0.0) last = e;
            }
            L.tok = last >= 0 ? last : 0;
        }
        __syncthreads();
        if (L.tok == 0x7FFFFFFF) return 0;
    }
    const int tok = L.tok;
    __syncthreads();
    return tok;
}

// ---------------------------------------------------------------- sequence

// Padding-free compaction fused into the sampler ("EMS-SD: Efficient
// Multi-sample Speculative Decoding", abstract: samples that accept different
// numbers of tokens are handled without padding).  Called by every thread of
// the workgroup that has just made sequence b's tokens final (n accepted
// drafts, out_tokens written with coherent stores): it appends the new KV rows
// q0 .. q0+n after the sequence's cache rows, advances kv_len[b] by e = n + 1
// and counts the sequence in; the last sequence to arrive writes cu_tokens
// (exclusive scan of e) and packs every sequence's e emitted tokens.  The same
// results as spec_compact_kv after the sampler.
template <int NT>
__device__ void compact_sequence(const AcceptParams& p, int b, int q0, int n, int* flag, int* scan) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int e = n + 1;
    const int L = p.kv_len[b];
    const long long start = p.kv_start[b];
    __syncthreads();  // every thread has read kv_len[b]
    if (tid == 0) {
        p.kv_len[b] = L + e;
        st_coh(p.cmp_e + b, e);
    }
    // arrive before the row copy: the packing needs the tokens and counts of
    // every sequence, not the copied rows (those are read by later launches)
    const bool last = arrive_last(p.cmp_cnt, p.B, flag);
    const size_t rb = static_cast<size_t>(p.row_bytes);
    const size_t dst0 = static_cast<size_t>(start + L) * rb, src0 = static_cast<size_t>(q0) * rb;
    const size_t nbytes = static_cast<size_t>(e) * rb;
    if (rb % 16 == 0) {
        const uint4* ks = reinterpret_cast<const uint4*>(p.k_new + src0);
        const uint4* vs = reinterpret_cast<const uint4*>(p.v_new + src0);
        uint4* kd = reinterpret_cast<uint4*>(p.k_cache + dst0);
        uint4* vd = reinterpret_cast<uint4*>(p.v_cache + dst0);
        for (size_t i = tid; i < nbytes / 16; i += NT) {
            const uint4 kv = ks[i], vv = vs[i];
            kd[i] = kv;
            vd[i] = vv;
        }
    } else {
        const uint32_t* ks = reinterpret_cast<const uint32_t*>(p.k_new + src0);
        const uint32_t* vs = reinterpret_cast<const uint32_t*>(p.v_new + src0);
        uint32_t* kd = reinterpret_cast<uint32_t*>(p.k_cache + dst0);
        uint32_t* vd = reinterpret_cast<uint32_t*>(p.v_cache + dst0);
        for (size_t i = tid; i < nbytes / 4; i += NT) {
            const uint32_t kv = ks[i], vv = vs[i];
            kd[i] = kv;
            vd[i] = vv;
        }
    }
    if (!last) return;
    // ---- the last sequence: thread t takes the sequences [t per, (t+1) per)
    const int per = (p.B + NT - 1) / NT;
    const int b0 = min(p.B, tid * per), b1 = min(p.B, b0 + per);
    int mine = 0;
    for (int bb = b0; bb < b1; ++bb) mine += ld_coh(p.cmp_e + bb);
    const int inc = wave_incl_scan(mine, lane);
    if (lane == 63) scan[wv] = inc;
    __syncthreads();
    int cu = 0, total = 0;
#pragma unroll
    for (int u = 0; u < NT / 64; ++u) {
        const int t = scan[u];
        cu += (u < wv) ? t : 0;
        total += t;
    }
    cu += inc - mine;
    for (int bb = b0; bb < b1; ++bb) {
        const int eb = ld_coh(p.cmp_e + bb);
        const int qb = seq_q0(p, bb);
        p.cu_tokens[bb] = cu;
        // the tokens eight at a time, their loads issued together
        for (int i0 = 0; i0 < eb; i0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = (i0 + u < eb) ? ld_coh(p.out_tokens + qb + i0 + u) : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u < eb) p.tokens_packed[cu + i0 + u] = v[u];
        }
        cu += eb;
    }
    if (tid == 0) p.cu_tokens[p.B] = total;
}

// Arrival of unit j of sequence b (all threads call it).  The units count
// themselves in seq_word[b] (top bits) and set bit j there when x_j was
// rejected; the last one to arrive stops at the first rejection n (K_b if
// none) and writes out_tokens (drafts before n, the token drawn at n, -1
// after it) and n_accepted.  A unit that drew a token stores it in utok first,
// and its store completes before its arrival.  Draft lengths above kMaskBits
// gather their rejection bits in seq_mask[b] instead.  has_tok: the token at
// n is known here (with no filter the draw kernel writes it).
__device__ __forceinline__ void sequence_arrival(const AcceptParams& p, int u, int b, int q0, int kb, int j,
                                                 bool rej, bool drew, int token, bool has_tok, MergeLds& L) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        if (drew) st_coh(p.utok + u, token);
        unsigned long long bits = 0ull;
        bool last;
        if (kb <= kMaskBits) {
            const unsigned long long add = kArrive | (rej ? (1ull << j) : 0ull);
            __builtin_amdgcn_s_waitcnt(0);
            const unsigned long long old =
                __hip_atomic_fetch_add(p.seq_word + b, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (old >> kMaskBits) == static_cast<unsigned long long>(kb);
            bits = (old + add) & (kArrive - 1);
        } else {
            if (rej) __hip_atomic_fetch_or(p.seq_mask + b, 1ull << j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);
            const unsigned long long old =
                __hip_atomic_fetch_add(p.seq_word + b, kArrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (old >> kMaskBits) == static_cast<unsigned long long>(kb);
            if (last) bits = ld_coh(p.seq_mask + b);
        }
        int n = -1;
        if (last) {
            n = bits ? __ffsll(bits) - 1 : kb;
            st_coh(p.seq_word + b, 0ull);
            if (kb > kMaskBits) st_coh(p.seq_mask + b, 0ull);
        }
        L.seqn = n;
    }
    __syncthreads();
    const int n = L.seqn;
    if (n < 0) return;
    if (tid <= kb) {
        // coherent stores: with the compaction on, another workgroup packs them
        int v = -1;
        bool st = true;
        if (tid < n) {
            v = p.draft_tokens[q0 - b + tid];
        } else if (tid == n) {
            st = has_tok;
            if (has_tok) v = (n == j) ? token : ld_coh(p.utok + q0 + n);
        }
        if (st) st_coh(p.out_tokens + q0 + tid, v);
    }
    if (tid == 0) {
        p.n_accepted[b] = n;
        st_coh(&p.seqs[b].n, n);
    }
    // the draw kernel writes the token at n without a filter: it compacts then
    if (p.compact && has_tok) compact_sequence<kMThreads>(p, b, q0, n, &L.cflag, L.cscan);
}

__device__ __forceinline__ DrawRows draw_rows(const MergeLds& L, bool residual) {
    const RowPart& T = L.r[0];
    const RowPart& D = L.r[1];
    DrawRows Rw;
    Rw.mq = T.m;
    Rw.tq = T.tau;
    Rw.Sq = T.kept;
    Rw.mp = residual ? D.m : T.m;
    Rw.tp = residual ? D.tau : T.tau;
    Rw.Sp = residual ? D.kept : T.kept;
    return Rw;
}

// ---------------------------------------------------------------- merge kernel

// One workgroup per unit u: the target row (first half of the workgroup) and,
// for j < K_b, the draft row (second half); then the accept test of x_j, the
// draw after a rejection or for the bonus row, and the unit's arrival at its
// sequence.
__global__ __launch_bounds__(kMThreads) void merge_kernel(AcceptParams p) {
    __shared__ MergeLds L;
    const int tid = threadIdx.x, lane = tid & 63;
    const int u = blockIdx.x;
    if (u >= p.nt) return;
    // sequence of unit u: the number of sequences whose rows all precede it
    int b;
    if (p.cu_q) {
        int cnt = 0;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int i = b0 + lane;
            cnt += __popcll(__ballot(i < p.B && p.cu_q[i + 1] <= u));
        }
        b = min(__builtin_amdgcn_readfirstlane(cnt), p.B - 1);
    } else {
        b = u / (p.K + 1);
    }
    const int q0 = seq_q0(p, b), kb = seq_kb(p, b), j = u - q0;
    const bool has_d = !p.greedy && j < kb;
    const int dr = p.nt + u - b;
    const int x = (j < kb) ? p.draft_tokens[u - b] : -1;
    const bool x_ok = x >= 0 && x < p.V;

    if (p.greedy) {
        fill_exp_table(L.tab);
        // argmax of the target row: the segment maxima, lowest index on ties
        if (tid < 64) {
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF;
            for (int s = lane; s < p.nseg; s += 64) {
                const SegHead* h = p.seg + static_cast<size_t>(u) * p.nseg + s;
                const float v = h->m;
                const int i = h->top;
                const bool take = (v > bv) | ((v == bv) & (i < bi));
                bv = take ? v : bv;
                bi = take ? i : bi;
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
                bv = take ? ov : bv;
                bi = take ? oi : bi;
            }
            if (lane == 0) L.tok = bi;
        }
        __syncthreads();
        const int am = L.tok;
        bool acc = true;
        if (j < kb) {
            if (tid == 0 && !x_ok) set_status(p.status, 1);
            acc = x_ok && x == am;
        }
        if (tid == 0) p.rows[u].argmax = am;
        const bool drew = (j == kb) || !acc;
        sequence_arrival(p, u, b, q0, kb, j, (j < kb) && !acc, drew, am, true, L);
        return;
    }

    const int rr = tid / kHalf, rt = tid & (kHalf - 1), rw = rt >> 6;
    RowPart& R = L.r[rr];
    const bool act = (rr == 0) || has_d;
    const int row = rr ? dr : u;
    const int nslots = p.nseg * p.klist;
    const bool lists = p.filter && p.nseg <= kListSegMax && nslots <= kHalf * kSlots;
    unsigned long long e[kSlots];
    float zpv[kSlots];

    // ---- one round trip: segment heads, listed bin masses and counts, the
    // drafted logit, the uniforms, then the list slots of this thread
    // (coalesced: slot rt + kHalf*i).  The segment kernel wrote them; this
    // launch reads them with plain loads.  Every load is issued before the
    // first LDS store; the list slots, issued last and first used by the
    // boundary-bin gather, arrive while the row statistics are formed.
    constexpr int kBmIter = (kListSegMax * kQB + kHalf - 1) / kHalf;
    static_assert(kMaxSeg <= kHalf, "one segment head per thread");
    SegHead h{};
    double bmv[kBmIter];
    int bcv[kBmIter];
    const int nb = (lists && act) ? p.nseg * kQB : 0;
    {
        const SegHead* hs = p.seg + static_cast<size_t>(row) * p.nseg;
        if (act && rt < p.nseg && !p.prestats) h = hs[rt];
        const double* bmr = p.bmass + static_cast<size_t>(row) * p.nseg * kQB;
        const int* bcr = p.bcnt + static_cast<size_t>(row) * p.nseg * kQB;
#pragma unroll
        for (int it = 0; it < kBmIter; ++it) {
            const int i = rt + kHalf * it;
            bmv[it] = (i < nb) ? bmr[i] : 0.0;
            bcv[it] = (i < nb && p.top_k > 0) ? bcr[i] : 0;
        }
    }
    // the drafted token's logit (with LM-head statistics there is no segment
    // pass to pick it up: read it from the row)
    const float zxv = !act ? 0.0f
                           : (p.prestats ? (x_ok && j < kb ? load1(row_ptr(p, row), p.bf16, x) : 0.0f)
                                         : p.zx[row]);
    const float uav = (tid == kMThreads - 1 && j < kb) ? p.u_accept[u - b] : 0.0f;
    const float usv = (tid == kMThreads - 1) ? p.u_sample[b] : 0.0f;
    {
        const unsigned long long* lb = p.list + static_cast<size_t>(row) * nslots;
        const float* zb = p.lzp + static_cast<size_t>(u) * nslots;
        const bool ldz = lists && rr == 0 && has_d;
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int f = rt + kHalf * i;
            const bool in = lists && act && f < nslots;
            e[i] = in ? lb[f] : 0ull;
            zpv[i] = (in && ldz) ? zb[f] : 0.0f;
        }
    }
    if (act) {
        if (rt < p.nseg) {
            R.seg_m[rt] = h.m;
            R.seg_top[rt] = h.top;
            R.seg_ocut[rt] = h.ocut;
            R.seg_n[rt] = h.n;
            R.seg_S[rt] = h.S;
        }
#pragma unroll
        for (int it = 0; it < kBmIter; ++it) {
            const int i = rt + kHalf * it;
            if (i < nb) {
                (&R.bm[0][0])[i] = bmv[it];
                if (p.top_k > 0) (&R.bc[0][0])[i] = bcv[it];
            }
        }
        if (rt == 0) R.zx = (x_ok && j < kb) ? zxv : 0.0f;
    }
    if (tid == kMThreads - 1) {
        L.ua = uav;
        L.us = usv;
    }
    fill_exp_table(L.tab);
    __syncthreads();

    // ---- row max, normaliser and bin masses in one step: every wave of a row
    // finds the row max and the segment scales exp((m_s - m)/T) itself (lane
    // l holds segments l and l + 64) and sums its share of the segments' listed
    // bin masses (every kRW-th segment; lane = row bin); the first wave also
    // the normaliser and the bins listed in every segment
    static_assert(kMaxSeg <= 128, "two segments per lane");
    if (act && p.prestats) {
        // no filter: the row's max and normaliser from the LM head's parts.
        // Every wave of the row finds the max over all parts; each adds the
        // rescaled sums of every kRW-th stretch of 64 parts (the waves'
        // shares are added in wave order after the barrier below).
        const size_t pr = rr ? static_cast<size_t>(dr - p.nt) : static_cast<size_t>(u);
        const float* pm = p.pre_m[rr] + pr * p.pre_parts;
        const double* ps = p.pre_s[rr] + pr * p.pre_parts;
        float m = -INFINITY;
        for (int i = lane; i < p.pre_parts; i += 64) m = fmaxf(m, pm[i]);
        m = wave_max(m);
        double Sacc = 0.0;
        for (int i = rt; i < p.pre_parts; i += kHalf) {
            const float mi = pm[i];
            if (mi != -INFINITY) Sacc += ps[i] * weight(mi, m, p.yscale, L.tab);
        }
        Sacc = wave_sum(Sacc);
        if (lane == 0) R.part[rw][0] = Sacc;
        if (rw == 0 && lane == 0) {
            R.m = m;
            R.top = qbin(m, p.qscale);
            R.ocmax = -1;
            R.fast = 0;
            R.tau = -INFINITY;
            R.zk = -INFINITY;
            R.zmin = -INFINITY;
            R.ccount = 0;
            R.needsub = 0;
            R.above = 0.0;
            R.abovec = 0;
        }
    } else if (act) {
        const bool s0 = lane < p.nseg, s1 = lane + 64 < p.nseg;
        const float v0 = s0 ? R.seg_m[lane] : -INFINITY;
        const float v1 = s1 ? R.seg_m[lane + 64] : -INFINITY;
        const float m = wave_max(fmaxf(v0, v1));
        const int top = qbin(m, p.qscale);
        const double sc0 = (v0 == -INFINITY) ? 0.0 : weight(v0, m, p.yscale, L.tab);
        const double sc1 = (v1 == -INFINITY) ? 0.0 : weight(v1, m, p.yscale, L.tab);
        if (rw == 0) {
            double Sacc = (s0 ? R.seg_S[lane] * sc0 : 0.0) + (s1 ? R.seg_S[lane + 64] * sc1 : 0.0);
            int oc = 0x7FFFFFFF;
            if (v0 != -INFINITY) oc = R.seg_ocut[lane] + (top - R.seg_top[lane]);
            if (v1 != -INFINITY) oc = min(oc, R.seg_ocut[lane + 64] + (top - R.seg_top[lane + 64]));
            Sacc = wave_sum(Sacc);
            oc = wave_min_i(oc);
            if (lane == 0) {
                R.m = m;
                R.top = top;
                R.S = Sacc;
                R.ocmax = oc;
                R.fast = lists ? 1 : 0;
                R.tau = -INFINITY;
                R.kept = Sacc;
                R.zk = -INFINITY;
                R.Sk = Sacc;
                R.zmin = -INFINITY;
                R.ccount = 0;
                R.needsub = 0;
                R.above = 0.0;
                R.abovec = 0;
            }
        }
        if (lists) {
            const int o = lane;
            double pm = 0.0;
            int pc = 0;
            for (int s = rw; s < p.nseg; s += kRW) {  // s is uniform
                const double scs = (s < 64) ? lane_read_d(sc0, s) : lane_read_d(sc1, s - 64);
                const int os = o - (top - R.seg_top[s]);
                if (R.seg_m[s] != -INFINITY && os >= 0 && os <= R.seg_ocut[s]) {
                    pm += R.bm[s][os] * scs;
                    if (p.top_k > 0) pc += R.bc[s][os];
                }
            }
            R.part[rw][o] = pm;
            R.cpart[rw][o] = pc;
        }
    }
    if (rw == 1) {  // the sub-bins start cleared
        R.sbm[lane] = 0.0;
        R.sbk[0][lane] = 0xFFFFFFFFu;
        R.sbk[1][lane] = 0u;
    }
    __syncthreads();
    if (p.prestats) {  // uniform: the normaliser from the waves' shares
        if (act && rw == 0 && lane == 0) {
            double Sr = 0.0;
#pragma unroll
            for (int w2 = 0; w2 < kRW; ++w2) Sr += R.part[w2][0];
            R.S = Sr;
            R.kept = Sr;
            R.Sk = Sr;
        }
        __syncthreads();
    }

    // valid slots of this thread: slot < its segment's list length
    unsigned vmask = 0u;
    if (lists && act) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int f = rt + kHalf * i;
            int sg, o;
            slot_pos(f, p.klist, &sg, &o);
            if (f < nslots && o < R.seg_n[min(sg, kMaxSeg - 1)]) vmask |= 1u << i;
        }
    }
    if (lists) {
        // ---- the first wave of a row adds the partial bin masses in a fixed
        // order and finds the first boundary bin (the top-k count boundary, or
        // the nucleus mass boundary)
        if (act && rw == 0) {
            const int o = lane;
            double mass = 0.0;
            int cnt = 0;
#pragma unroll
            for (int w2 = 0; w2 < kRW; ++w2) {
                mass += R.part[w2][o];
                cnt += R.cpart[w2][o];
            }
            R.mass[o] = mass;
            int og;
            if (p.top_k > 0) {
                const int cum = wave_incl_scan(cnt, lane);
                const unsigned long long hit = __ballot(cum >= p.top_k);
                og = hit ? __ffsll(hit) - 1 : -1;
                const int before = __shfl(cum, max(og - 1, 0), 64);
                if (lane == 0) R.abovec = og > 0 ? before : 0;
            } else {
                const double target = p.top_p * R.S;
                const double cum = wave_incl_scan(mass, lane);
                const unsigned long long hit = __ballot(cum >= target);
                og = hit ? __ffsll(hit) - 1 : -1;
                const double before = __shfl(cum, max(og - 1, 0), 64);
                if (lane == 0) R.above = og > 0 ? before : 0.0;
            }
            if (lane == 0) {
                R.og = og;
                if (!(og >= 0 && og <= R.ocmax)) R.fast = 0;
                if (p.top_k == 0 && R.fast) {
                    R.target = p.top_p * R.S;
                    R.needsub = 1;
                }
            }
        }
        __syncthreads();
        // ---- top-k: rank the count boundary bin; the k-th largest z, the
        // mass of the top-k set, and where its nucleus boundary lies
        if (p.top_k > 0) {  // uniform
            rank_bin(p, e, vmask, act, L);
            if (act && rw == 0 && R.fast) {
                const int n = R.ccount;
                const float zk = R.rk.rz[min(max(p.top_k - R.abovec - 1, 0), n - 1)];
                const double mv = (lane < R.og) ? R.mass[lane] : 0.0;
                const double cum = wave_incl_scan(mv, lane);
                const double above = __shfl(cum, 63, 64);  // the complete bins above og
                double part = 0.0;
                for (int c0 = 0; c0 < n; c0 += 64) {
                    const int i = c0 + lane;
                    part += (i < n && R.rk.rz[i] >= zk) ? R.rk.rw[i] : 0.0;
                }
                part = wave_sum(part);
                const double Sk = above + part;
                if (p.top_p < 1.0) {
                    const double target = p.top_p * Sk;
                    const unsigned long long hit = __ballot(lane < R.og && cum >= target);
                    const int on = hit ? __ffsll(hit) - 1 : 0;
                    const double before = __shfl(cum, max(on - 1, 0), 64);
                    if (lane == 0) {
                        if (hit) {  // in a bin above og: all of it lies above zk
                            R.og = on;
                            R.above = on > 0 ? before : 0.0;
                        } else {    // in og itself, among the entries with z >= zk
                            R.above = above;
                            R.zmin = zk;
                        }
                        R.target = target;
                        R.needsub = 1;
                    }
                } else if (lane == 0) {
                    R.tau = zk;
                    R.kept = Sk;
                }
            }
            __syncthreads();
        }
        subbin_threshold(p, e, vmask, L);
    }

    // ---- rows whose lists cannot decide: radix select over the whole row;
    // such a unit draws from the whole target row (the slot registers are
    // dead from here on that path)
    if (p.filter && (!L.r[0].fast || (has_d && !L.r[1].fast))) {  // uniform
        for (int r2 = 0; r2 < 2; ++r2) {
            RowPart& Q = L.r[r2];
            if (r2 == 1 && !has_d) break;
            if (Q.fast) continue;  // uniform
            const RadixRow rrow{row_ptr(p, r2 ? dr : u), p.V, p.bf16, p.vec, p.yscale};
            const float m = Q.m;
            float zk = -INFINITY;
            double Sk = Q.S;
            if (p.top_k > 0) {
                radix_threshold(rrow, m, 0.0, p.top_k, -INFINITY, L);
                zk = L.tau;
                Sk = L.kept;
            }
            if (p.top_p < 1.0) radix_threshold(rrow, m, p.top_p * Sk, 0, zk, L);
            if (tid == 0) {
                Q.tau = (p.top_p < 1.0) ? L.tau : zk;
                Q.kept = (p.top_p < 1.0) ? L.kept : Sk;
            }
            __syncthreads();
        }
        const bool acc = accept_test(p, u, dr, j, kb, x_ok, L);
        const bool need = (j == kb) || !acc;
        int token = -1;
        if (need) {  // uniform
            const bool residual = j < kb;
            const FullRow fr{row_ptr(p, u), row_ptr(p, residual ? dr : u), p.status, p.V, p.bf16, p.yscale};
            token = draw_full_row(fr, draw_rows(L, residual), residual, L.us, L);
        }
        sequence_arrival(p, u, b, q0, kb, j, (j < kb) && !acc, need, token, true, L);
        return;
    }
    if (lists) {  // uniform: the lists hold both rows' kept sets
        // the draw -- needed after a rejection, or for the bonus row -- is
        // made together with the accept test instead of after it
        const bool residual = j < kb;
        const DrawRows Rw = draw_rows(L, residual);
        AcceptIn ai{};
        if (tid == kMThreads - 1) ai = accept_in(L);
        int token = draw_from_lists(p, Rw, residual, L.us, e, zpv, vmask, ai, u, dr, j, kb, x_ok, L);
        const bool acc = L.acc != 0;
        const bool need = (j == kb) || !acc;
        if (need && token < 0) {  // uniform: no residual mass
            const FullRow fr{row_ptr(p, u), row_ptr(p, residual ? dr : u), p.status, p.V, p.bf16, p.yscale};
            token = draw_full_row(fr, Rw, residual, L.us, L);
        }
        sequence_arrival(p, u, b, q0, kb, j, (j < kb) && !acc, need, token, true, L);
        return;
    }
    const bool acc = accept_test(p, u, dr, j, kb, x_ok, L);
    const bool need = (j == kb) || !acc;
    int token = -1;
    if (p.filter && need) {  // uniform: beyond the list path
        const bool residual = j < kb;
        const FullRow fr{row_ptr(p, u), row_ptr(p, residual ? dr : u), p.status, p.V, p.bf16, p.yscale};
        token = draw_full_row(fr, draw_rows(L, residual), residual, L.us, L);
    }
    sequence_arrival(p, u, b, q0, kb, j, (j < kb) && !acc, p.filter && need, token, p.filter != 0, L);
}

// ---------------------------------------------------------------- segment kernel

template <int EPT>
__global__ __launch_bounds__(kThreads) void segment_kernel(AcceptParams p) {
    __shared__ SegLds L;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int total = p.grid_units * p.nseg;
    const int logical = xcd_remap(blockIdx.x, total);
    const int u = logical / p.nseg, s = logical % p.nseg;
    if (u >= p.nt) return;
    // sequence of unit u: the number of sequences whose rows all precede it
    int b;
    if (p.cu_q) {
        int cnt = 0;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int i = b0 + lane;
            cnt += __popcll(__ballot(i < p.B && p.cu_q[i + 1] <= u));
        }
        b = min(__builtin_amdgcn_readfirstlane(cnt), p.B - 1);
    } else {
        b = u / (p.K + 1);
    }
    const int q0 = seq_q0(p, b), kb = seq_kb(p, b), j = u - q0;
    const bool has_d = !p.greedy && j < kb;
    const int dr = p.nt + u - b;
    float z[2][EPT];
    load_segment<EPT>(row_ptr(p, u), p.bf16, p.vec, p.V, s, tid, z[0]);
    if (has_d) {
        load_segment<EPT>(row_ptr(p, dr), p.bf16, p.vec, p.V, s, tid, z[1]);
    } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) z[1][k] = -INFINITY;
    }
    fill_exp_table(L.tab);
    // the segment counters start at zero (ordered before use by the first barrier)
    for (int i = tid; i < 2 * 4 * (kQB + 64); i += kThreads) (&L.hc[0][0][0])[i] = 0;
    for (int i = tid; i < 2 * kQB; i += kThreads) (&L.hm[0][0])[i] = 0.0;
    // the drafted token's logits, stored by the thread that holds them
    // (element k of thread t has id seg_lo + (k/4)*1024 + 4*t + k%4)
    const int x = (j < kb) ? p.draft_tokens[u - b] : -1;
    const int seg_lo = s * kThreads * EPT;
    if (!p.greedy && x >= seg_lo && x < seg_lo + kThreads * EPT && x < p.V) {
        const int off = x - seg_lo;
        const int kx = ((off >> 10) << 2) | (off & 3);
        if (tid == ((off & 1023) >> 2)) {
            float zq = 0.0f, zp = 0.0f;
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                zq = (k == kx) ? z[0][k] : zq;
                zp = (k == kx) ? z[1][k] : zp;
            }
            p.zx[u] = zq;
            if (has_d) p.zx[dr] = zp;
        }
    }

    if (p.greedy) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int e = seg_index<EPT>(s, tid, k);
            const bool take = (e < p.V) & ((z[0][k] > bv) | ((z[0][k] == bv) & (e < bi)));
            bv = take ? z[0][k] : bv;
            bi = take ? e : bi;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
        if (lane == 0) {
            L.gv[wv] = bv;
            L.gi[wv] = bi;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w2 = 1; w2 < kThreads / 64; ++w2)
                if (L.gv[w2] > bv || (L.gv[w2] == bv && L.gi[w2] < bi)) {
                    bv = L.gv[w2];
                    bi = L.gi[w2];
                }
            SegHead* h = p.seg + static_cast<size_t>(u) * p.nseg + s;
            h->m = bv;
            h->top = bi;
        }
    } else {
        float lm[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < EPT; ++k) lm[r] = fmaxf(lm[r], z[r][k]);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            lm[r] = wave_max(lm[r]);
            if (lane == 0) L.red_f[r][wv] = lm[r];
        }
        __syncthreads();
        float ms[2];
        int top[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            ms[r] = fmaxf(fmaxf(L.red_f[r][0], L.red_f[r][1]), fmaxf(L.red_f[r][2], L.red_f[r][3]));
            top[r] = qbin(ms[r], p.qscale);
        }
        // one pass per element: the fp64 weight (a row max of -inf gives NaN
        // arguments, which exp2_256 maps to 0) and, with a filter on, the bin
        // offset (kept) and its count
        double acc[2] = {0.0, 0.0};
        unsigned ow[2][EPT / 4];  // bin offsets (0..kQB-1 in the window, kQB.. below it), four per word
        const unsigned past = static_cast<unsigned>(kQB + lane);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int g = 0; g < EPT / 4; ++g) ow[r][g] = 0u;  // row 1 without a draft: never listed (ocut -1)
            if (r == 1 && !has_d) continue;  // uniform
            const double mr = static_cast<double>(ms[r]);
            if (p.filter) {  // uniform
#pragma unroll
                for (int k = 0; k < EPT; ++k) {
                    acc[r] += exp2_256((static_cast<double>(z[r][k]) - mr) * p.yscale, L.tab);
                    // the bin offset; below the window a counter past the bins
                    // (at most the lane's own: no branch, few conflicts)
                    const unsigned o = min(static_cast<unsigned>(top[r] - qbin(z[r][k], p.qscale)), past);
                    ow[r][k >> 2] |= o << (8 * (k & 3));
                    atomicAdd(&L.hc[r][wv][o], 1);
                    // four elements at a time: the exps of a whole row in
                    // flight at once would cost occupancy
                    if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int k = 0; k < EPT; ++k) {
                    acc[r] += exp2_256((static_cast<double>(z[r][k]) - mr) * p.yscale, L.tab);
                    if ((k & 7) == 7) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            acc[r] = wave_sum(acc[r]);
            if (lane == 0) L.red_d[r][wv] = acc[r];
        }
        __syncthreads();
        if (p.filter) segment_lists<EPT>(p, s, u, dr, has_d, z, ow, top, ms, L);
        if (tid < (has_d ? 2 : 1)) {
            const int r = tid;
            SegHead* h = p.seg + static_cast<size_t>(r ? dr : u) * p.nseg + s;
            h->S = (L.red_d[r][0] + L.red_d[r][1]) + (L.red_d[r][2] + L.red_d[r][3]);
            if (!p.filter) h->m = r ? ms[1] : ms[0];
        }
    }
}


// ---------------------------------------------------------------- draw (no filter)

struct DrawLds {
    double tab[256];
    double red_d[kThreads / 64];
    double red_d2[kThreads / 64];
    int flag;
    int cflag;                      // compaction: this sequence arrived last
    int cscan[kThreads / 64];       // compaction: per-wave scan totals
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
    const double wq = weight(zq, c.rq.m, p.yscale, c.tab) * c.invSq;
    const double q = (valid & (zq >= c.rq.tau)) ? wq : 0.0;
    *qv = q;
    if (c.residual) {
        const double wp = weight(zp, c.rp.m, p.yscale, c.tab) * c.invSp;
        const double pv = (valid & (zp >= c.rp.tau)) ? wp : 0.0;
        const double d = q - pv;
        *w = d > 0.0 ? d : 0.0;
    } else {
        *w = q;
    }
}

template <int EPT>
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
    // the stopping rows' logits and their records in one round trip
    const bool residual = n < K;
    const void* qrow = row_ptr(p, q0 + n);
    const void* prow = residual ? row_ptr(p, nt + q0 - b + n) : nullptr;
    float zq[EPT], zp[EPT];
    load_segment<EPT>(qrow, p.bf16, p.vec, p.V, s, tid, zq);
    if (residual) load_segment<EPT>(prow, p.bf16, p.vec, p.V, s, tid, zp);
    if (tid == 0) L.rr[0] = p.rows[q0 + n];
    if (tid == 1 && residual) L.rr[1] = p.rows[nt + q0 - b + n];
    __syncthreads();

    DrawCtx c;
    c.tab = L.tab;
    c.residual = residual;
    c.qrow = qrow;
    c.rq = L.rr[0];
    c.invSq = 1.0 / c.rq.S;
    if (residual) {
        c.prow = prow;
        c.rp = L.rr[1];
        c.invSp = 1.0 / c.rp.S;
    } else {
        c.prow = nullptr;
        c.rp = c.rq;
        c.invSp = 0.0;
    }
    double ws = 0.0, qs = 0.0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        double w, qv;
        const bool valid = seg_index<EPT>(s, tid, k) < p.V;
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
    for (int t = tid; t < p.nseg; t += kThreads) {
        L.ds[t] = ld_coh(p.dsum + static_cast<size_t>(b) * p.nseg + t);
        L.qs[t] = ld_coh(p.qsum + static_cast<size_t>(b) * p.nseg + t);
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
    // contiguous layout for the exact in-order scan: thread t owns EPT ids
    const int e0 = ss * (kThreads * EPT) + tid * EPT;
    float q4[EPT], p4[EPT];
#pragma unroll
    for (int i = 0; i < EPT / 4; ++i) {
        load4(c.qrow, p.bf16, p.vec, p.V, e0 + 4 * i, q4 + 4 * i);
        if (c.residual) load4(c.prow, p.bf16, p.vec, p.V, e0 + 4 * i, p4 + 4 * i);
    }
    double w[EPT];
    double loc = 0.0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
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
    for (int k = 0; k < EPT; ++k) {
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
        st_coh(p.out_tokens + q0 + n, tok);
    }
    if (p.compact) compact_sequence<kThreads>(p, b, q0, n, &L.cflag, L.cscan);
}

// ---------------------------------------------------------------- host

struct Layout {
    int nseg, klist;
};

Layout layout_for(int ept, int V) {
    const int seg = kThreads * ept;
    return Layout{(V + seg - 1) / seg, 16 * ept};
}

// Workgroups of one launch per compute unit, cached per device.
int device_cus() {
    static int cache[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 256;
    }
    if (cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    cache[dev] = cus;
    return cus;
}

// Segments of 4096 (EPT 16) or 3072 (EPT 12) logits: the list path needs
// nseg*klist <= 4096 slots and nseg <= kListSegMax; among the sizes that
// allow it (when a filter is on), the one whose grid fills the last round of
// workgroups on the compute units best (three resident per unit).
int choose_ept(long long units, int V, bool filter) {
    const int cus = device_cus();
    int best = 16;
    double best_fill = -1.0;
    for (int ept : {16, 12}) {
        const Layout l = layout_for(ept, V);
        const bool lists = l.nseg <= kListSegMax && l.nseg * l.klist <= kHalf * kSlots;
        if (filter && !lists && best_fill >= 0.0) continue;
        const long long wgs = units * l.nseg;
        const long long slots = 3LL * cus;
        const long long rounds = (wgs + slots - 1) / slots;
        const double fill = static_cast<double>(wgs) / static_cast<double>(rounds * slots);
        const bool better = best_fill < 0.0 || fill > best_fill + 1e-9;
        const Layout bl = layout_for(best, V);
        const bool best_lists = bl.nseg <= kListSegMax && bl.nseg * bl.klist <= kHalf * kSlots;
        if (better || (filter && lists && !best_lists)) {
            best = ept;
            best_fill = fill;
        }
    }
    return best;
}

// Offsets of the workspace parts (counters first: their place depends on B only).
struct WsParts {
    size_t seq_word, seq_mask, draw_cnt, cmp_cnt, cmp_e, seg, list, lzp, bmass, bcnt, rows, zx, utok, seqs,
        dsum, qsum, end;
};

WsParts ws_parts(int B, long long nt, int V) {
    size_t nseg = 0, slots = 0;
    for (int ept : {16, 12}) {
        const Layout l = layout_for(ept, V);
        nseg = nseg > static_cast<size_t>(l.nseg) ? nseg : static_cast<size_t>(l.nseg);
        const size_t sl = static_cast<size_t>(l.nseg) * l.klist;
        slots = slots > sl ? slots : sl;
    }
    const size_t nrows = static_cast<size_t>(2 * nt - B);  // target and draft rows
    WsParts w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        off = (off + 255) & ~static_cast<size_t>(255);
        const size_t at = off;
        off += bytes;
        return at;
    };
    w.seq_word = take(static_cast<size_t>(B) * sizeof(unsigned long long));
    w.seq_mask = take(static_cast<size_t>(B) * sizeof(unsigned long long));
    w.draw_cnt = take(static_cast<size_t>(B) * sizeof(int));
    w.cmp_cnt = take(sizeof(int));
    w.cmp_e = take(static_cast<size_t>(B) * sizeof(int));
    w.seg = take(nrows * nseg * sizeof(SegHead));
    w.list = take(nrows * slots * sizeof(unsigned long long));
    w.lzp = take(static_cast<size_t>(nt) * slots * sizeof(float));
    w.bmass = take(nrows * nseg * kQB * sizeof(double));
    w.bcnt = take(nrows * nseg * kQB * sizeof(int));
    w.rows = take(nrows * sizeof(RowRec));
    w.zx = take(nrows * sizeof(float));
    w.utok = take(static_cast<size_t>(nt) * sizeof(int));
    w.seqs = take(static_cast<size_t>(B) * sizeof(SeqRec));
    w.dsum = take(static_cast<size_t>(B) * nseg * sizeof(double));
    w.qsum = take(static_cast<size_t>(B) * nseg * sizeof(double));
    w.end = (off + 255) & ~static_cast<size_t>(255);
    return w;
}

}  // namespace

size_t accept_workspace_bytes(int B, long long nt, int V) { return ws_parts(B, nt, V).end; }

int accept_max_vocab() { return 262144; }
int accept_max_drafts() { return kMaxDrafts; }

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
    p.bf16 = a.bf16;
    p.vec = (a.V % 4 == 0) ? 1 : 0;
    p.greedy = a.greedy;
    p.top_k = (!a.greedy && a.top_k > 0 && a.top_k < a.V) ? a.top_k : 0;
    p.filter = (!a.greedy && (a.top_p < 1.0f || p.top_k > 0)) ? 1 : 0;
    p.yscale = (1.0 / static_cast<double>(a.temperature)) * kY256PerLn2;
    p.top_p = static_cast<double>(a.top_p);
    p.qscale = static_cast<float>(4.0 / static_cast<double>(a.temperature));
    const int ept = choose_ept(a.nt, a.V, p.filter != 0);
    const Layout lay = layout_for(ept, a.V);
    p.nseg = lay.nseg;
    p.klist = lay.klist;
    p.grid_units = (a.nt + 7) / 8 * 8;

    const WsParts w = ws_parts(a.B, a.nt, a.V);
    char* base = static_cast<char*>(a.workspace);
    p.seq_word = reinterpret_cast<unsigned long long*>(base + w.seq_word);
    p.seq_mask = reinterpret_cast<unsigned long long*>(base + w.seq_mask);
    p.draw_cnt = reinterpret_cast<int*>(base + w.draw_cnt);
    p.cmp_cnt = reinterpret_cast<int*>(base + w.cmp_cnt);
    p.cmp_e = reinterpret_cast<int*>(base + w.cmp_e);
    p.compact = a.kv_len ? 1 : 0;
    p.kv_len = a.kv_len;
    p.kv_start = a.kv_start;
    p.k_cache = static_cast<char*>(a.k_cache);
    p.v_cache = static_cast<char*>(a.v_cache);
    p.k_new = static_cast<const char*>(a.k_new);
    p.v_new = static_cast<const char*>(a.v_new);
    p.tokens_packed = a.tokens_packed;
    p.cu_tokens = a.cu_tokens;
    p.row_bytes = static_cast<long long>(a.row_bytes);
    p.seg = reinterpret_cast<SegHead*>(base + w.seg);
    p.list = reinterpret_cast<unsigned long long*>(base + w.list);
    p.lzp = reinterpret_cast<float*>(base + w.lzp);
    p.bmass = reinterpret_cast<double*>(base + w.bmass);
    p.bcnt = reinterpret_cast<int*>(base + w.bcnt);
    p.rows = reinterpret_cast<RowRec*>(base + w.rows);
    p.zx = reinterpret_cast<float*>(base + w.zx);
    p.utok = reinterpret_cast<int*>(base + w.utok);
    p.seqs = reinterpret_cast<SeqRec*>(base + w.seqs);
    p.dsum = reinterpret_cast<double*>(base + w.dsum);
    p.qsum = reinterpret_cast<double*>(base + w.qsum);

    p.prestats = (a.pre_m[0] && !p.filter && !p.greedy) ? 1 : 0;
    p.pre_m[0] = a.pre_m[0];
    p.pre_m[1] = a.pre_m[1];
    p.pre_s[0] = a.pre_s[0];
    p.pre_s[1] = a.pre_s[1];
    p.pre_parts = a.pre_parts;
    hipError_t err = hipSuccess;
    if (!p.prestats) {  // the LM head's statistics replace the segment pass
        const dim3 grid(p.grid_units * p.nseg);
        if (ept == 16)
            hipLaunchKernelGGL(segment_kernel<16>, grid, dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL(segment_kernel<12>, grid, dim3(kThreads), 0, stream, p);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(merge_kernel, dim3(a.nt), dim3(kMThreads), 0, stream, p);
    err = hipGetLastError();
    if (err != hipSuccess || a.greedy || p.filter) return err;
    const int grid_seqs = (a.B + 7) / 8 * 8;
    if (ept == 16)
        hipLaunchKernelGGL(draw_kernel<16>, dim3(grid_seqs * p.nseg), dim3(kThreads), 0, stream, p, grid_seqs);
    else
        hipLaunchKernelGGL(draw_kernel<12>, dim3(grid_seqs * p.nseg), dim3(kThreads), 0, stream, p, grid_seqs);
    return hipGetLastError();
}

}  // namespace sv
