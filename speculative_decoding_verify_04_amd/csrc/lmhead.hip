// LM head with the sampler's row statistics in its epilogue, on gfx950.
//
// Method: "Accelerating Large Language Model Decoding with Speculative
// Sampling", section "Conditional scoring": the target model scores the K
// drafts and one more position in a single call, and its last linear layer
// turns each row's final hidden state into logits over the vocabulary.  The
// sampler's first need from every row is its maximum and its normaliser
// (section "Modified rejection sampling": q and p are softmax distributions,
// tempered first).  This kernel computes the logits
//   z[r][v] = sum_h hidden[r][h] * W[v][h]      (bf16 inputs, fp32 accumulation)
// and, while they are still on chip, every row's statistics over each part of
// kPart consecutive vocabulary ids:
//   m_p = max z,   S_p = sum exp((z - m_p) / T)   (fp64, exp2_256 of sv_math.h)
// so that a sampler without a filter can take each row's max and normaliser
// from the parts (m = max m_p, S = sum S_p exp((m_p - m)/T)) instead of
// reading the logits a second time.
//
// lm_head_kernel<NR, KU>: one workgroup (4 waves) per (part of kPart = 64
//   ids, block of 16 NR rows).  The hidden dimension is split into 4
//   contiguous ranges of 32-wide steps, one per wave, so each wave keeps
//   4 weight tiles of 16 ids x 32 in flight per step (KU steps are loaded
//   before their products).  Every step is v_mfma_f32_16x16x32_bf16 with the
//   weight tile as the A operand (a lane loads 8 consecutive bf16 of one
//   weight row) and the hidden rows as the B operand (8 consecutive bf16 of
//   one hidden row): logits^T = W hidden^T.  The 4 waves' partial sums meet in
//   LDS (wave w owns id tile w); then each wave stores its 16 ids of every row
//   (16-byte stores) and the part's max and fp64 sum are reduced by lane
//   exchanges and LDS.
//   Launch order: block L runs on XCD L mod 8; the row blocks of one part are
//   consecutive on one XCD, so the part's weight slice is fetched from HBM
//   once and served to the other row blocks from that XCD's L2.  The weight
//   matrix is streamed once; the hidden rows stay in L2.
//   Used for up to 16 rows (one row tile; the weight stream bounds it).
//
// lm_gemm_rows_kernel<RT>: 17 to 64 rows, still bound by the weight stream.
//   One workgroup (3 waves) per tile of 192 ids; both the block of 16 RT
//   rows and the weight tile pass through LDS as below, so each hidden
//   element loaded feeds 192 products; each wave holds one statistics part
//   of all the rows.
//
// lm_gemm_kernel: more rows, where the products bound the call.  One
//   workgroup (8 waves) per (block of 192 rows, tile of 256 ids = four
//   statistics parts); both operands pass through LDS in 32-wide steps of the
//   hidden dimension, five stages deep (direct 16-byte global-to-LDS loads,
//   one barrier per step), so each weight and hidden element read from L2 or
//   HBM feeds 256 or 192 products instead of 64.  Wave (wr, wn) computes rows
//   96 wr .. +96 and ids 64 wn .. +64 of the tile: 24 products
//   v_mfma_f32_16x16x32_bf16 per step, the weight tile as A, the hidden rows
//   as B, as above.  Each wave then holds a whole statistics part of its
//   rows, so the epilogue needs no exchange between waves.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_math.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kPart = 64;      // vocabulary ids per workgroup (and per statistics part)
constexpr int kXcd = 8;        // blocks are dealt to the XCDs round-robin

struct LmParams {
    const uint16_t* hidden;  // [rows][H] bf16
    const uint16_t* weight;  // [V][H] bf16
    float* logits;           // [rows][V]
    float* part_m;           // [rows][nparts]
    double* part_s;          // [rows][nparts]
    int rows, H, V, nparts, nrb;   // nrb: row blocks of 16 NR rows
    double ys;               // 256 / (T ln 2)
};

template <int NR>
struct LmLds {
    double tab[256];
    floatx4 red[4][3][NR][64];  // [owner tile][other wave][row tile][lane] partial sums
    float m[4][NR][16];         // per-wave row maxima of the part
    double s[4][NR][16];        // per-wave row sums relative to the part max
};

template <int NR, int KU>
__global__ __launch_bounds__(kThreads) void lm_head_kernel(LmParams p) {
    __shared__ LmLds<NR> S;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col16 = lane & 15, kg = lane >> 4;
    // XCD-aware order: the row blocks of a part are consecutive on one XCD
    const int L = blockIdx.x;
    const int xcd = L % kXcd, i = L / kXcd;
    const int part = (i / p.nrb) * kXcd + xcd;
    const int rb = i % p.nrb;
    if (part >= p.nparts) return;  // uniform: the whole workgroup leaves
    const int v0 = part * kPart;
    const int r0 = rb * 16 * NR;
    S.tab[tid] = exp2(static_cast<double>(tid) * (1.0 / 256.0));

    // operand rows of this lane (clamped: ids past V and rows past `rows`
    // compute values that are never stored)
    const uint16_t* wrow[4];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
        const int v = min(v0 + vt * 16 + col16, p.V - 1);
        wrow[vt] = p.weight + static_cast<size_t>(v) * p.H + kg * 8;
    }
    const uint16_t* hrow[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        const int r = min(r0 + t * 16 + col16, p.rows - 1);
        hrow[t] = p.hidden + static_cast<size_t>(r) * p.H + kg * 8;
    }

    floatx4 acc[4][NR];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
        for (int t = 0; t < NR; ++t) acc[vt][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // this wave's 32-wide steps of the hidden dimension (H is a multiple of
    // 32, checked on the host): [nst w / 4, nst (w+1) / 4)
    const int nst = p.H >> 5;
    const int s1 = (nst * (w + 1)) >> 2;
    int s = (nst * w) >> 2;
    for (; s + KU <= s1; s += KU) {
        bf16x8 a[KU][4], bb[KU][NR];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int h = (s + u) * 32;
#pragma unroll
            for (int vt = 0; vt < 4; ++vt) a[u][vt] = *reinterpret_cast<const bf16x8*>(wrow[vt] + h);
#pragma unroll
            for (int t = 0; t < NR; ++t) bb[u][t] = *reinterpret_cast<const bf16x8*>(hrow[t] + h);
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int vt = 0; vt < 4; ++vt)
#pragma unroll
                for (int t = 0; t < NR; ++t)
                    acc[vt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][vt], bb[u][t], acc[vt][t], 0, 0, 0);
    }
    for (; s < s1; ++s) {
        const int h = s * 32;
        bf16x8 a[4], bb[NR];
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) a[vt] = *reinterpret_cast<const bf16x8*>(wrow[vt] + h);
#pragma unroll
        for (int t = 0; t < NR; ++t) bb[t] = *reinterpret_cast<const bf16x8*>(hrow[t] + h);
#pragma unroll
        for (int vt = 0; vt < 4; ++vt)
#pragma unroll
            for (int t = 0; t < NR; ++t)
                acc[vt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[vt], bb[t], acc[vt][t], 0, 0, 0);
    }

    // ---- the 4 waves' partial sums meet: wave w owns id tile w; the others
    // leave their share of it in LDS (slot: the writer's rank among the
    // three non-owners), and the owner adds all four in wave order
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
        if (vt != w) {
            const int slot = w < vt ? w : w - 1;
#pragma unroll
            for (int t = 0; t < NR; ++t) S.red[vt][slot][t][lane] = acc[vt][t];
        }
    }
    __syncthreads();
    floatx4 z[NR];
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
        if (vt == w) {  // uniform
#pragma unroll
            for (int t = 0; t < NR; ++t) z[t] = acc[vt][t];
        }
    }
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        floatx4 sum = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int src = 0; src < 4; ++src) {
            floatx4 x;
            if (src == w) {
                x = z[t];
            } else {
                x = S.red[w][src < w ? src : src - 1][t][lane];
            }
            sum += x;
        }
        z[t] = sum;
    }

    // ---- epilogue: lane holds (row r0 + 16 t + col16, ids v0 + 16 w + 4 kg + e)
    const int vb = v0 + w * 16 + kg * 4;
    float mx[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        const int r = r0 + t * 16 + col16;
        if (r < p.rows) {
            float* dst = p.logits + static_cast<size_t>(r) * p.V + vb;
            if (vb + 3 < p.V && (p.V & 3) == 0) {
                *reinterpret_cast<float4*>(dst) = make_float4(z[t][0], z[t][1], z[t][2], z[t][3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (vb + e < p.V) dst[e] = z[t][e];
            }
        }
        mx[t] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (vb + e < p.V) mx[t] = fmaxf(mx[t], z[t][e]);
        // over the 4 id groups of the wave (lanes col16, +16, +32, +48)
        mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], 16, 64));
        mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], 32, 64));
        if (kg == 0) S.m[w][t][col16] = mx[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        const float m = fmaxf(fmaxf(S.m[0][t][col16], S.m[1][t][col16]),
                              fmaxf(S.m[2][t][col16], S.m[3][t][col16]));
        double sum = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (vb + e < p.V)
                sum += exp2_256((static_cast<double>(z[t][e]) - static_cast<double>(m)) * p.ys, S.tab);
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        if (kg == 0) S.s[w][t][col16] = sum;
        mx[t] = m;
    }
    __syncthreads();
    if (w == 0 && kg == 0) {
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int r = r0 + t * 16 + col16;
            if (r < p.rows) {
                const size_t o = static_cast<size_t>(r) * p.nparts + part;
                p.part_m[o] = mx[t];
                p.part_s[o] = (S.s[0][t][col16] + S.s[1][t][col16]) + (S.s[2][t][col16] + S.s[3][t][col16]);
            }
        }
    }
}

constexpr int kGK = 32;        // hidden-dimension step: one 16x16x32 product
constexpr int kStreamRows = 16; // up to this many rows: lm_head_kernel
constexpr int kSmallRows = 64;  // up to this many rows: lm_gemm_rows_kernel

// One stage of both operand tiles: rows of 32 bf16 (four 16-byte chunks);
// chunk c of row r is stored at c ^ gemm_swz(r), so that the 16-byte operand
// reads of 16 consecutive rows (one chunk each) fall on distinct banks: any
// 8 consecutive rows cover all eight 16-byte bank groups of 128 bytes, and
// rows r, r+4, r+8, r+12 all four positions of their 64-byte group.
__device__ __forceinline__ int gemm_swz(int r) { return ((r >> 1) ^ ((r >> 3) & 1)) & 3; }

template <int GM, int GN>
struct GemmStage {
    uint4 h[GM * kGK / 8];   // hidden rows of the block (GM / 16 KiB)
    uint4 w[GN * kGK / 8];   // weight rows of the tile (GN / 16 KiB)
};

// s_waitcnt immediate for vmcnt(n), n < 64 (the other counters left alone)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Tile of GM = WR RT 16 rows x GN = WN 64 ids, WR x WN waves, each wave RT
// row tiles x 4 id tiles (one statistics part), NST stages.  (The body is a
// device function called by plain kernels: as a kernel template it would not
// get its host-side launch stub, because the direct LDS load builtin does
// not instantiate in the host pass.)
template <int WR, int RT, int WN, int NST>
__device__ __forceinline__ void lm_gemm_body(const LmParams& p, int ntiles) {
    constexpr int GM = WR * RT * 16;
    constexpr int GN = WN * 64;
    constexpr int NW = WR * WN;                 // waves
    constexpr int TH = GM / 16, TW = GN / 16;   // loads of 64 x 16 bytes per stage: hidden, weight
    constexpr int TI = TH + TW;
    constexpr int LPW = (TI + NW - 1) / NW;     // loads per wave and stage (the excess repeats loads)
    static_assert(NST >= 3 && NST <= 6 && (NST - 2) * LPW < 64, "stages and the wait count");
    // NST separate LDS objects (the unused ones are not allocated): the
    // compiler's wait for one stage's direct loads then does not cover the
    // others
    __shared__ GemmStage<GM, GN> G0, G1, G2, G3, G4, G5;
    __shared__ double tab[256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col16 = lane & 15, kg = lane >> 4;
    const int wr = w / WN, wn = w % WN;
    // XCD-aware order: the row blocks of an id tile are consecutive on one XCD
    const int L = blockIdx.x;
    const int xcd = L % kXcd, i = L / kXcd;
    const int tile = (i / p.nrb) * kXcd + xcd;
    const int rb = i % p.nrb;
    if (tile >= ntiles) return;  // uniform: the whole workgroup leaves
    const int id0 = tile * GN;
    const int row0 = rb * GM;
    for (int t = tid; t < 256; t += NW * 64) tab[t] = exp2(static_cast<double>(t) * (1.0 / 256.0));
    __syncthreads();  // the table, before any load is in flight

    // this wave's loads of a stage: load q = (w LPW + j) mod TI (the last
    // waves may repeat loads of the first ones: same data to the same place,
    // so that every wave issues as many); loads q < TH carry hidden chunks
    // q*64 + lane, the others weight chunks (q - TH)*64 + lane; chunk c is
    // row c/4 at stored position c%4, i.e. logical chunk (c%4) ^ gemm_swz(row).
    // Rows past `rows` and ids past V are clamped (their products are never
    // stored).
    const uint16_t* src[LPW];
    int dst[LPW];
    bool ish[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int q = (w * LPW + j) % TI;
        ish[j] = q < TH;
        const int qq = ish[j] ? q : q - TH;
        const int r = (qq * 64 + lane) >> 2;
        const int c = (lane & 3) ^ gemm_swz(r);
        src[j] = ish[j] ? p.hidden + static_cast<size_t>(min(row0 + r, p.rows - 1)) * p.H + c * 8
                        : p.weight + static_cast<size_t>(min(id0 + r, p.V - 1)) * p.H + c * 8;
        dst[j] = qq * 64;
    }
    const int nk = p.H / kGK;
    // steps past the last re-read the last one into a stage no longer read,
    // so that every step issues the same loads (the compiler's waits then
    // follow the explicit counts below).  The stage objects are named
    // directly, so the direct-load builtin sees LDS addresses; st folds to a
    // constant in every use.
    auto dma = [&](const uint16_t* g, bool h, int d, int st) __attribute__((always_inline)) {
        if (h) {
            if (st == 0) __builtin_amdgcn_global_load_lds(g, G0.h + d, 16, 0, 0);
            else if (st == 1) __builtin_amdgcn_global_load_lds(g, G1.h + d, 16, 0, 0);
            else if (st == 2) __builtin_amdgcn_global_load_lds(g, G2.h + d, 16, 0, 0);
            else if (st == 3) __builtin_amdgcn_global_load_lds(g, G3.h + d, 16, 0, 0);
            else if (st == 4) __builtin_amdgcn_global_load_lds(g, G4.h + d, 16, 0, 0);
            else __builtin_amdgcn_global_load_lds(g, G5.h + d, 16, 0, 0);
        } else {
            if (st == 0) __builtin_amdgcn_global_load_lds(g, G0.w + d, 16, 0, 0);
            else if (st == 1) __builtin_amdgcn_global_load_lds(g, G1.w + d, 16, 0, 0);
            else if (st == 2) __builtin_amdgcn_global_load_lds(g, G2.w + d, 16, 0, 0);
            else if (st == 3) __builtin_amdgcn_global_load_lds(g, G3.w + d, 16, 0, 0);
            else if (st == 4) __builtin_amdgcn_global_load_lds(g, G4.w + d, 16, 0, 0);
            else __builtin_amdgcn_global_load_lds(g, G5.w + d, 16, 0, 0);
        }
    };
    auto issue = [&](int k, int st) __attribute__((always_inline)) {
        const int k0 = min(k, nk - 1) * kGK;
#pragma unroll
        for (int j = 0; j < LPW; ++j) dma(src[j] + k0, ish[j], dst[j], st);
    };

    floatx4 acc[4][RT];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[it][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // operand reads: row base + col16, logical chunk kg (stored at
    // kg ^ gemm_swz(col16): the bases are multiples of 16)
    const int loff = col16 * 4 + (kg ^ gemm_swz(col16));
    auto compute = [&](const GemmStage<GM, GN>& G) __attribute__((always_inline)) {
        bf16x8 wa[4], hb[RT];
#pragma unroll
        for (int it = 0; it < 4; ++it)
            wa[it] = *reinterpret_cast<const bf16x8*>(&G.w[(wn * 64 + it * 16) * 4 + loff]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            hb[rt] = *reinterpret_cast<const bf16x8*>(&G.h[((wr * RT + rt) * 16) * 4 + loff]);
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                acc[it][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[it], hb[rt], acc[it][rt], 0, 0, 0);
    };
    // step k (in stage st = k mod NST): this wave's loads of step k are in
    // when at most those of steps k+1 .. k+NST-2 are in flight; the barrier
    // makes every wave's loads of step k visible and frees the stage of step
    // k - 1 for step k + NST - 1 (every wave's reads of it fed its products
    // before it arrived).  A plain barrier: the workgroup release of
    // __syncthreads would also wait for the later steps' loads; the LDS-only
    // acquire keeps the reads after it.
    auto step = [&](int k, int st) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * LPW));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        issue(k + NST - 1, (st + NST - 1) % NST);
        if (st == 0) compute(G0);
        else if (st == 1) compute(G1);
        else if (st == 2) compute(G2);
        else if (st == 3) compute(G3);
        else if (st == 4) compute(G4);
        else compute(G5);
    };
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) issue(s, s);
    int k = 0;
    for (; k + NST <= nk; k += NST) {
#pragma unroll
        for (int s = 0; s < NST; ++s) step(k + s, s);
    }
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (k + s < nk) step(k + s, s);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load outlives the loop

    // ---- epilogue: acc[it][rt][e] is row row0 + 16 (RT wr + rt) + col16, id
    // id0 + 64 wn + 16 it + 4 kg + e; this wave holds part WN tile + wn of its
    // rows whole
    const int part = tile * WN + wn;
    const int vw = id0 + wn * 64 + kg * 4;
    const bool vec = (p.V & 3) == 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + (wr * RT + rt) * 16 + col16;
        if (r < p.rows) {
            float* dstp = p.logits + static_cast<size_t>(r) * p.V;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int vb = vw + it * 16;
                if (vec && vb + 3 < p.V) {
                    *reinterpret_cast<float4*>(dstp + vb) =
                        make_float4(acc[it][rt][0], acc[it][rt][1], acc[it][rt][2], acc[it][rt][3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (vb + e < p.V) dstp[vb + e] = acc[it][rt][e];
                }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (vw + it * 16 + e < p.V) mx = fmaxf(mx, acc[it][rt][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        double sum = 0.0;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (vw + it * 16 + e < p.V)
                    sum += exp2_256((static_cast<double>(acc[it][rt][e]) - static_cast<double>(mx)) * p.ys, tab);
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        if (kg == 0 && r < p.rows && part < p.nparts) {
            const size_t o = static_cast<size_t>(r) * p.nparts + part;
            p.part_m[o] = mx;
            p.part_s[o] = sum;
        }
    }
}

// Decode row counts (weight-stream bound): 16 RT rows x 192 ids, 3 waves of
// RT row tiles x 64 ids, six stages (one workgroup per CU; with V = 49152 the
// 256 tiles are one per CU).  The hidden rows are a small share of each
// workgroup's loads next to its 192 weight rows.
constexpr int kRowsGN = 192, kRowsThreads = 192;
template <int RT>
__global__ __launch_bounds__(192, 1) void lm_gemm_rows_kernel(LmParams p, int ntiles) {
    lm_gemm_body<1, RT, 3, 6>(p, ntiles);
}
// More rows (product bound): 192 rows x 256 ids, 8 waves of 96 rows x 64 ids,
// five stages (140 KiB, one workgroup per CU).
constexpr int kGM = 192, kGN = 256, kGThreads = 512;
__global__ __launch_bounds__(512, 1) void lm_gemm_kernel(LmParams p, int ntiles) {
    lm_gemm_body<2, 6, 4, 5>(p, ntiles);
}

}  // namespace

int lm_head_parts(int V) { return (V + kPart - 1) / kPart; }
int lm_head_part_len() { return kPart; }

hipError_t lm_head_launch(const LmArgs& a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    LmParams p{};
    p.hidden = static_cast<const uint16_t*>(a.hidden);
    p.weight = static_cast<const uint16_t*>(a.weight);
    p.logits = a.logits;
    p.part_m = a.part_max;
    p.part_s = a.part_sum;
    p.rows = a.rows;
    p.H = a.H;
    p.V = a.V;
    p.nparts = lm_head_parts(a.V);
    p.ys = (1.0 / static_cast<double>(a.temperature)) * kY256PerLn2;
    if (a.rows <= kStreamRows) {
        // one row tile: 64-id parts, the weight streamed by 4 waves
        p.nrb = 1;
        // every XCD gets ceil(nparts / 8) parts' worth of workgroups; those of
        // parts past the end leave at once
        const int blocks = ((p.nparts + kXcd - 1) / kXcd) * kXcd;
        hipLaunchKernelGGL((lm_head_kernel<1, 2>), dim3(blocks), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    // row blocks x id tiles; every XCD gets ceil(ntiles / 8) tiles' worth of
    // workgroups, those past the end leave at once
    const bool big = a.rows > kSmallRows;
    const int rt = (a.rows + 15) / 16;  // up to 64 rows: one row block of rt row tiles
    const int gm = big ? kGM : 16 * rt, gn = big ? kGN : kRowsGN;
    const int ntiles = (a.V + gn - 1) / gn;
    p.nrb = (a.rows + gm - 1) / gm;
    const int blocks = ((ntiles + kXcd - 1) / kXcd) * kXcd * p.nrb;
    if (big)
        hipLaunchKernelGGL(lm_gemm_kernel, dim3(blocks), dim3(kGThreads), 0, stream, p, ntiles);
    else if (rt == 2)
        hipLaunchKernelGGL(lm_gemm_rows_kernel<2>, dim3(blocks), dim3(kRowsThreads), 0, stream, p, ntiles);
    else if (rt == 3)
        hipLaunchKernelGGL(lm_gemm_rows_kernel<3>, dim3(blocks), dim3(kRowsThreads), 0, stream, p, ntiles);
    else
        hipLaunchKernelGGL(lm_gemm_rows_kernel<4>, dim3(blocks), dim3(kRowsThreads), 0, stream, p, ntiles);
    return hipGetLastError();
}

}  // namespace sv
