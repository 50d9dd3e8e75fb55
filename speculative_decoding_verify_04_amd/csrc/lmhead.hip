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

template <int NR, int KU>
void launch_nr(const LmParams& p, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL((lm_head_kernel<NR, KU>), dim3(blocks), dim3(kThreads), 0, stream, p);
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
    const int tiles = (a.rows + 15) / 16;
    const int nr = tiles < 4 ? tiles : 4;
    p.nrb = (tiles + nr - 1) / nr;
    // every XCD gets ceil(nparts / 8) parts' worth of workgroups; those of
    // parts past the end leave at once
    const int blocks = ((p.nparts + kXcd - 1) / kXcd) * kXcd * p.nrb;
    switch (nr) {
        case 1: launch_nr<1, 2>(p, blocks, stream); break;
        case 2: launch_nr<2, 2>(p, blocks, stream); break;
        case 3: launch_nr<3, 2>(p, blocks, stream); break;
        default: launch_nr<4, 2>(p, blocks, stream); break;
    }
    return hipGetLastError();
}

}  // namespace sv
