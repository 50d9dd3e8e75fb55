// Modified rejection sampling for a batch of verify rounds on gfx950.
//
// Method: "Accelerating Large Language Model Decoding with Speculative
// Sampling", section "Modified rejection sampling" and Theorem 1: accept draft
// x_j with probability min(1, q(x_j)/p(x_j)) left to right, resample the first
// rejected position from (q - p)_+, draw a bonus token from the last target
// row when all K drafts pass; temperature and nucleus modify q and p first.
//
// Kernels (one launch each, chained inside a launch by last-arriver counters):
//   rows_kernel  grid = rows x segments.  Each workgroup reads one 4096-logit
//                segment once, computes its max, its fp64 mass relative to
//                that max, and (nucleus) an fp64 mass histogram over absolute
//                quarter-unit bins of z/T.  The last segment of a row to finish
//                merges the row: max, normaliser S, nucleus threshold (exact:
//                the boundary bin is re-read and its few candidates sorted;
//                a radix select over the row handles every other case), and
//                the fp64 weight of the drafted token.  The last row of a
//                sequence to finish runs the accept scan.
//                Every merge first fetches all it needs with independent
//                loads issued together (one memory round trip), then works
//                from LDS: a chain of dependent global loads costs ~0.3 us
//                per link on MI355X.
//   draw_kernel  grid = sequences x segments.  fp64 residual (q'-p')_+ or
//                bonus q' weights of the stopping row, per-segment sums; the
//                last segment picks the crossing segment and scans it exactly.
// Every quantity that decides a token is fp64; the exp of the logits is the
// table-driven fp64 exp of sv_math.h (table of 2^(j/64) built per workgroup).
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_math.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kSeg = kThreads * kPerThread;  // 4096 logits per segment
constexpr int kBins = 128;                   // nucleus histogram bins (width 0.25 in z/T)
constexpr int kCap = 1024;                   // boundary-bin candidates sorted in LDS
constexpr int kMaxSeg = 64;                  // V <= 64 * 4096
constexpr int kMaxRowsPerSeq = 2 * 64 + 1;   // K <= 64

struct SegHead {
    float m;      // segment max (greedy: max value)
    int kb_top;   // bin of the max (greedy: index of the max)
    double S;     // sum of exp((z - m)/T) over the segment
};

struct RowRec {
    float m;      // row max
    float tau;    // nucleus threshold logit (-inf: no nucleus)
    double S;     // kept mass relative to m (= full normaliser without nucleus)
    double wx;    // exp((z[x] - m)/T) for the drafted token x of this row
    int kept;     // drafted token inside the nucleus
    int argmax;   // lowest id of the row maximum (greedy)
    int pad0, pad1;
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
    double* hmass;
    int* hcnt;
    RowRec* rows;
    SeqRec* seqs;
    double* dsum;
    double* qsum;
    int* row_cnt;
    int* seq_cnt;
    int* draw_cnt;
    int B, K, V, nseg, nrows, grid_rows;
    int bf16, vec, nucleus, greedy;
    double invT;
    double top_p;
    float bscale;  // 4 / T: bin index of z is floor(z * bscale)
};

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
    const int nt = p.B * (p.K + 1);
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
    double hm[kBins];
    int hc[kBins];
    double red_d[kThreads / 64];
    float red_f[kThreads / 64];
    int flag;
    // row merge
    float seg_m[kMaxSeg];
    int seg_kb[kMaxSeg];
    double seg_S[kMaxSeg];
    double sc[kMaxSeg];       // per-segment rescale exp((m_s - m)/T)
    float m;
    int argmax;
    double S;
    float zx;                 // logit of the drafted token of the row
    // nucleus threshold
    double rh_m[256];         // radix-select digit masses
    int rh_c[256];
    float cz[kCap];
    int cidx[kCap];
    double cw[kCap];
    int ccount;
    int bsel;
    double above;
    float tau;
    double kept;
    int mode;                 // 0: candidate path, 1: radix fallback
    uint32_t prefix, mask;
    int chosen;
    // sequence scan
    RowRec rr[kMaxRowsPerSeq];
    float ua[64];
    int x[64];
};

// Exact tie-closed nucleus threshold by radix select over the whole row
// (4 passes of 8 bits over order-preserving keys, fp64 digit masses).  Used
// only when the boundary bin is unusable (deep threshold or flat rows).
__device__ void radix_threshold(const AcceptParams& p, const void* row, float m, double target,
                                RowsLds& L) {
    const int tid = threadIdx.x;
    if (tid == 0) { L.prefix = 0; L.mask = 0; L.above = 0.0; }
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int d = tid; d < 256; d += kThreads) { L.rh_m[d] = 0.0; L.rh_c[d] = 0; }
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
                if (e < p.V && (key & mask) == prefix) {
                    const int d = (key >> shift) & 0xFF;
                    atomicAdd(&L.rh_m[d], weight(z[k], m, p.invT, L.tab));
                    atomicAdd(&L.rh_c[d], 1);
                }
            }
        }
        __syncthreads();
        if (tid == 0) {
            double cum = L.above;
            int chosen = -1, lowest = -1;
            for (int d = 255; d >= 0; --d) {
                if (L.rh_c[d] == 0) continue;
                lowest = d;
                if (cum + L.rh_m[d] >= target) { chosen = d; break; }
                cum += L.rh_m[d];
            }
            if (chosen < 0) {  // rounding left the target unreached: keep everything
                chosen = lowest;
                cum -= L.rh_m[lowest];
            }
            L.above = cum;
            L.prefix |= static_cast<uint32_t>(chosen) << shift;
            L.mask |= 0xFFu << shift;
            L.chosen = chosen;
        }
        __syncthreads();
    }
    if (tid == 0) {
        L.tau = fkey_inv(L.prefix);
        L.kept = L.above + L.rh_m[L.chosen];
    }
    __syncthreads();
}

// Bitonic sort of L.cz/L.cidx[0, n2) by (z descending, id ascending).
__device__ void sort_candidates(RowsLds& L, int n2) {
    const int tid = threadIdx.x;
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n2 / 2; i += kThreads) {
                int a = 2 * i - (i & (stride - 1));
                int b = a + stride;
                bool desc_block = ((a & size) == 0);
                float za = L.cz[a], zb = L.cz[b];
                int ia = L.cidx[a], ib = L.cidx[b];
                bool a_first = (za > zb) || (za == zb && ia < ib);
                if (a_first != desc_block) {
                    L.cz[a] = zb; L.cz[b] = za;
                    L.cidx[a] = ib; L.cidx[b] = ia;
                }
            }
            __syncthreads();
        }
    }
}

// Exact nucleus threshold of one row from its merged histogram: the boundary
// bin's elements are gathered by one pass over the row (batched loads), sorted
// by (z desc, id asc) and scanned until the kept mass reaches the target.
__device__ void nucleus_threshold(const AcceptParams& p, int r, const void* row, float m,
                                  double S, RowsLds& L) {
    const int tid = threadIdx.x;
    const double target = p.top_p * S;
    const int kb_top = bin_of(m, p.bscale);
    // merged histogram over bins kb_top - og, og in [0, kBins): thread og sums
    // the segments in fixed order, four independent loads at a time
    if (tid < kBins) {
        double hm = 0.0;
        int hc = 0;
        for (int s0 = 0; s0 < p.nseg; s0 += 4) {
            double vm[4];
            int vc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + u;
                const int o = (s < p.nseg) ? tid - (kb_top - L.seg_kb[s]) : -1;
                const bool ok = (s < p.nseg) && o >= 0 && o < kBins && L.sc[s] != 0.0;
                const size_t h = (static_cast<size_t>(r) * p.nseg + (ok ? s : 0)) * kBins + (ok ? o : 0);
                vm[u] = ok ? ld_coh(p.hmass + h) : 0.0;
                vc[u] = ok ? ld_coh(p.hcnt + h) : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (s0 + u < p.nseg) {
                    hm += vm[u] * L.sc[s0 + u];
                    hc += vc[u];
                }
            }
        }
        L.hm[tid] = hm;
        L.hc[tid] = hc;
    }
    __syncthreads();
    if (tid == 0) {
        double cum = 0.0;
        int bsel = -1;
        for (int og = 0; og < kBins; ++og) {
            if (cum + L.hm[og] >= target) { bsel = og; break; }
            cum += L.hm[og];
        }
        L.bsel = bsel;
        L.above = cum;
        L.mode = (bsel < 0 || L.hc[bsel] > kCap) ? 1 : 0;
        L.ccount = 0;
    }
    __syncthreads();
    if (L.mode == 0) {
        const int kb_sel = kb_top - L.bsel;
        // one pass over the row, 8 independent 16-byte loads per thread in flight
        for (int base = 0; base < p.V; base += kThreads * 32) {
            float z[32];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                load4(row, p.bf16, p.vec, p.V, base + (i * kThreads + tid) * 4, z + 4 * i);
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                const int e = base + ((k >> 2) * kThreads + tid) * 4 + (k & 3);
                if (e < p.V && bin_of(z[k], p.bscale) == kb_sel) {
                    const int slot = atomicAdd(&L.ccount, 1);
                    if (slot < kCap) { L.cz[slot] = z[k]; L.cidx[slot] = e; }
                }
            }
        }
        __syncthreads();
        const int n = L.ccount;
        if (n > kCap || n == 0) {
            if (tid == 0) L.mode = 1;
        } else {
            int n2 = 1;
            while (n2 < n) n2 <<= 1;
            for (int i = n + tid; i < n2; i += kThreads) {
                L.cz[i] = -INFINITY;
                L.cidx[i] = 0x7FFFFFFF;
            }
            __syncthreads();
            sort_candidates(L, n2);
            for (int i = tid; i < n; i += kThreads) L.cw[i] = weight(L.cz[i], m, p.invT, L.tab);
            __syncthreads();
            // first sorted candidate whose running mass reaches the target
            if (tid < 64) {
                const int lane = tid;
                double run = L.above;
                int istar = -1;
                for (int c0 = 0; c0 < n && istar < 0; c0 += 64) {
                    const double v = (c0 + lane < n) ? L.cw[c0 + lane] : 0.0;
                    const double inc = run + wave_incl_scan(v, lane);
                    const unsigned long long hit = __ballot(c0 + lane < n && inc >= target);
                    if (hit) istar = c0 + __ffsll(hit) - 1;
                    run = __shfl(inc, 63, 64);
                }
                if (istar < 0) istar = n - 1;
                const float tau = L.cz[istar];
                // kept mass: everything above the bin plus candidates >= tau
                double part = 0.0;
                for (int c0 = 0; c0 < n; c0 += 64) {
                    const int i = c0 + lane;
                    part += (i < n && L.cz[i] >= tau) ? L.cw[i] : 0.0;
                }
                part = wave_sum(part);
                if (lane == 0) {
                    L.tau = tau;
                    L.kept = L.above + part;
                }
            }
            __syncthreads();
        }
    }
    __syncthreads();
    if (L.mode == 1) radix_threshold(p, row, m, target, L);
}

// Merge the segments of row r and write its RowRec.
__device__ void finalize_row(const AcceptParams& p, int r, RowsLds& L) {
    const int tid = threadIdx.x;
    const int nt = p.B * (p.K + 1);
    const void* row = row_ptr(p, r);
    const SegHead* sr = p.seg + static_cast<size_t>(r) * p.nseg;

    // drafted token of this row: target row j < K, or draft row j
    int j = -1, b = 0;
    if (r < nt) {
        b = r / (p.K + 1);
        j = r % (p.K + 1);
        if (j == p.K) j = -1;
    } else {
        b = (r - nt) / p.K;
        j = (r - nt) % p.K;
    }
    int x = -1;
    if (j >= 0) x = p.draft_tokens[b * p.K + j];
    const bool x_ok = (x >= 0 && x < p.V);

    // one round trip: segment heads (one per thread) and the drafted logit
    if (tid < p.nseg) {
        L.seg_m[tid] = ld_coh(&sr[tid].m);
        L.seg_kb[tid] = ld_coh(&sr[tid].kb_top);
        L.seg_S[tid] = ld_coh(&sr[tid].S);
    }
    if (tid == kThreads - 1) L.zx = (j >= 0 && x_ok && !p.greedy) ? load1(row, p.bf16, x) : 0.0f;
    __syncthreads();
    if (tid == 0) {
        float m = -INFINITY;
        int arg = 0;
        for (int s = 0; s < p.nseg; ++s)
            if (L.seg_m[s] > m) { m = L.seg_m[s]; arg = L.seg_kb[s]; }
        L.m = m;
        L.argmax = arg;
    }
    __syncthreads();
    const float m = L.m;

    RowRec rec;
    rec.m = m;
    rec.tau = -INFINITY;
    rec.argmax = L.argmax;
    rec.kept = 1;
    rec.wx = 0.0;
    rec.S = 0.0;
    rec.pad0 = rec.pad1 = 0;

    if (!p.greedy) {
        if (tid < p.nseg) {
            const float ms = L.seg_m[tid];
            L.sc[tid] = (ms == -INFINITY) ? 0.0 : weight(ms, m, p.invT, L.tab);
        }
        __syncthreads();
        if (tid == 0) {
            double S = 0.0;
            for (int s = 0; s < p.nseg; ++s) S += L.seg_S[s] * L.sc[s];
            L.S = S;
        }
        __syncthreads();
        rec.S = L.S;
        if (p.nucleus) {
            nucleus_threshold(p, r, row, m, L.S, L);
            rec.tau = L.tau;
            rec.S = L.kept;
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
    }
}

// Accept scan of sequence b once all of its rows are final.
__device__ void finalize_sequence(const AcceptParams& p, int b, RowsLds& L) {
    const int tid = threadIdx.x;
    const int K = p.K, nt = p.B * (K + 1);
    const int nr = p.greedy ? K + 1 : 2 * K + 1;
    // one round trip: the sequence's row records, drafts and uniforms
    if (tid < nr) {
        const int r = (tid <= K) ? b * (K + 1) + tid : nt + b * K + (tid - K - 1);
        const RowRec* src = p.rows + r;
        L.rr[tid].m = ld_coh(&src->m);
        L.rr[tid].tau = ld_coh(&src->tau);
        L.rr[tid].S = ld_coh(&src->S);
        L.rr[tid].wx = ld_coh(&src->wx);
        L.rr[tid].kept = ld_coh(&src->kept);
        L.rr[tid].argmax = ld_coh(&src->argmax);
    }
    if (tid >= 128 && tid - 128 < K) {
        L.x[tid - 128] = p.draft_tokens[b * K + tid - 128];
        L.ua[tid - 128] = p.greedy ? 0.0f : p.u_accept[b * K + tid - 128];
    }
    __syncthreads();
    if (tid != 0) return;
    int n = K;
    for (int jj = 0; jj < K; ++jj) {
        bool acc;
        const RowRec& tr = L.rr[jj];
        if (p.greedy) {
            acc = (L.x[jj] == tr.argmax);
        } else {
            const RowRec& dr = L.rr[K + 1 + jj];
            const double q = tr.kept ? tr.wx / tr.S : 0.0;
            const double pp = dr.kept ? dr.wx / dr.S : 0.0;
            const float u = L.ua[jj];
            if (!(u >= 0.0f && u < 1.0f)) set_status(p.status, 2);
            acc = (pp > 0.0) ? (static_cast<double>(u) * pp < q) : (q > 0.0);
        }
        if (!acc) { n = jj; break; }
    }
    int32_t* out = p.out_tokens + static_cast<size_t>(b) * (K + 1);
    for (int i = 0; i < n; ++i) out[i] = L.x[i];
    for (int i = n + 1; i <= K; ++i) out[i] = -1;
    if (p.greedy) out[n] = L.rr[n].argmax;
    p.n_accepted[b] = n;
    p.seqs[b].n = n;
}

__global__ __launch_bounds__(kThreads) void rows_kernel(AcceptParams p) {
    __shared__ RowsLds L;
    const int tid = threadIdx.x;
    const int total = p.grid_rows * p.nseg;
    const int logical = xcd_remap(blockIdx.x, total);
    const int r = logical / p.nseg, s = logical % p.nseg;
    if (r >= p.nrows) return;
    const void* row = row_ptr(p, r);

    float z[kPerThread];
    load_segment(row, p.bf16, p.vec, p.V, s, tid, z);
    fill_exp_table(L.tab);
    __syncthreads();

    if (p.greedy) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            int e = seg_index(s, tid, k);
            if (e < p.V && (z[k] > bv || (z[k] == bv && e < bi))) { bv = z[k]; bi = e; }
        }
        // (value desc, index asc) reduction
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
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
        double w[kPerThread];
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            w[k] = (ms == -INFINITY) ? 0.0 : weight(z[k], ms, p.invT, L.tab);
            acc += w[k];
        }
        const double Ss = block_sum<kThreads>(acc, L.red_d);
        const int kb_top = bin_of(ms, p.bscale);
        if (p.nucleus) {
            if (tid < kBins) { L.hm[tid] = 0.0; L.hc[tid] = 0; }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) {
                const int o = kb_top - bin_of(z[k], p.bscale);
                if (w[k] > 0.0 && o < kBins) {
                    atomicAdd(&L.hm[o], w[k]);
                    atomicAdd(&L.hc[o], 1);
                }
            }
            __syncthreads();
            if (tid < kBins) {
                const size_t h = (static_cast<size_t>(r) * p.nseg + s) * kBins + tid;
                st_coh(p.hmass + h, L.hm[tid]);
                st_coh(p.hcnt + h, L.hc[tid]);
            }
        }
        if (tid == 0) {
            SegHead* dst = p.seg + static_cast<size_t>(r) * p.nseg + s;
            st_coh(&dst->m, ms);
            st_coh(&dst->kb_top, kb_top);
            st_coh(&dst->S, Ss);
        }
    }

    if (!arrive_last(p.row_cnt + r, p.nseg, &L.flag)) return;
    finalize_row(p, r, L);

    const int nt = p.B * (p.K + 1);
    const int b = (r < nt) ? r / (p.K + 1) : (r - nt) / p.K;
    const int rows_per_seq = p.greedy ? p.K + 1 : 2 * p.K + 1;
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
    const double q = (valid && zq >= c.rq.tau) ? weight(zq, c.rq.m, p.invT, c.tab) * c.invSq : 0.0;
    *qv = q;
    if (c.residual) {
        const double pv = (valid && zp >= c.rp.tau) ? weight(zp, c.rp.m, p.invT, c.tab) * c.invSp : 0.0;
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
    const int K = p.K, nt = p.B * (K + 1);

    if (tid == 0) L.n = min(max(p.seqs[b].n, 0), K);
    fill_exp_table(L.tab);
    __syncthreads();
    const int n = L.n;
    if (tid == 0) L.rr[0] = p.rows[b * (K + 1) + n];
    if (tid == 1 && n < K) L.rr[1] = p.rows[nt + b * K + n];
    __syncthreads();

    DrawCtx c;
    c.tab = L.tab;
    c.residual = n < K;
    c.qrow = row_ptr(p, b * (K + 1) + n);
    c.rq = L.rr[0];
    c.invSq = 1.0 / c.rq.S;
    if (c.residual) {
        c.prow = row_ptr(p, nt + b * K + n);
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
        if (mine == 0x7FFFFFFF && w[k] > 0.0 && target < run) mine = e0 + k;
    }
    if (mine != 0x7FFFFFFF) atomicMin(&L.tok, mine);
    if (lastpos >= 0) atomicMax(&L.last_pos, lastpos);
    __syncthreads();
    if (tid == 0) {
        int tok = L.tok != 0x7FFFFFFF ? L.tok : L.last_pos;
        if (tok < 0) tok = 0;
        p.out_tokens[static_cast<size_t>(b) * (K + 1) + n] = tok;
    }
}

}  // namespace

size_t accept_workspace_bytes(int B, int K, int V) {
    const size_t nseg = (static_cast<size_t>(V) + kSeg - 1) / kSeg;
    const size_t nrows = static_cast<size_t>(B) * (2 * K + 1);
    size_t off = 0;
    auto take = [&](size_t bytes) { off = (off + 255) & ~static_cast<size_t>(255); off += bytes; };
    take(nrows * nseg * sizeof(SegHead));
    take(nrows * nseg * kBins * sizeof(double));
    take(nrows * nseg * kBins * sizeof(int));
    take(nrows * sizeof(RowRec));
    take(static_cast<size_t>(B) * sizeof(SeqRec));
    take(static_cast<size_t>(B) * nseg * sizeof(double));
    take(static_cast<size_t>(B) * nseg * sizeof(double));
    take(nrows * sizeof(int));
    take(static_cast<size_t>(B) * sizeof(int));
    take(static_cast<size_t>(B) * sizeof(int));
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
    p.V = a.V;
    p.nseg = (a.V + kSeg - 1) / kSeg;
    p.bf16 = a.bf16;
    p.vec = (a.V % 4 == 0) ? 1 : 0;
    p.greedy = a.greedy;
    p.nucleus = (!a.greedy && a.top_p < 1.0f) ? 1 : 0;
    p.invT = 1.0 / static_cast<double>(a.temperature);
    p.top_p = static_cast<double>(a.top_p);
    p.bscale = static_cast<float>(4.0 / static_cast<double>(a.temperature));
    p.nrows = a.greedy ? a.B * (a.K + 1) : a.B * (2 * a.K + 1);
    p.grid_rows = (p.nrows + 7) / 8 * 8;

    const size_t nseg = p.nseg;
    const size_t nrows_max = static_cast<size_t>(a.B) * (2 * a.K + 1);
    char* base = static_cast<char*>(a.workspace);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        off = (off + 255) & ~static_cast<size_t>(255);
        char* ptr = base + off;
        off += bytes;
        return ptr;
    };
    p.seg = reinterpret_cast<SegHead*>(take(nrows_max * nseg * sizeof(SegHead)));
    p.hmass = reinterpret_cast<double*>(take(nrows_max * nseg * kBins * sizeof(double)));
    p.hcnt = reinterpret_cast<int*>(take(nrows_max * nseg * kBins * sizeof(int)));
    p.rows = reinterpret_cast<RowRec*>(take(nrows_max * sizeof(RowRec)));
    p.seqs = reinterpret_cast<SeqRec*>(take(static_cast<size_t>(a.B) * sizeof(SeqRec)));
    p.dsum = reinterpret_cast<double*>(take(static_cast<size_t>(a.B) * nseg * sizeof(double)));
    p.qsum = reinterpret_cast<double*>(take(static_cast<size_t>(a.B) * nseg * sizeof(double)));
    p.row_cnt = reinterpret_cast<int*>(take(nrows_max * sizeof(int)));
    p.seq_cnt = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * sizeof(int)));
    p.draw_cnt = reinterpret_cast<int*>(take(static_cast<size_t>(a.B) * sizeof(int)));

    hipLaunchKernelGGL(rows_kernel, dim3(p.grid_rows * p.nseg), dim3(kThreads), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.greedy) return err;
    const int grid_seqs = (a.B + 7) / 8 * 8;
    hipLaunchKernelGGL(draw_kernel, dim3(grid_seqs * p.nseg), dim3(kThreads), 0, stream, p,
                       grid_seqs);
    return hipGetLastError();
}

}  // namespace sv
