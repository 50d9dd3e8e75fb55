// Padding-free compaction after a verify round, on gfx950.
//
// Method: "EMS-SD: Efficient Multi-sample Speculative Decoding" (abstract):
// samples accept different numbers of tokens in the verification phase; they
// are handled without padding tokens, so no extra memory or compute is spent.
// With e_b = n_b + 1 tokens emitted by sequence b ("Accelerating Large Language
// Model Decoding with Speculative Sampling", "Modified rejection sampling": at
// least one and at most K_b+1 tokens per round):
//   cu = exclusive scan of e;  packed[cu_b + i] = out_tokens[q_b + i];
//   cache rows L_b .. L_b + n_b of b <- new rows q_b .. q_b + n_b;  L_b += e_b,
// where q_b is the first row of sequence b: cu_q[b] with ragged draft lengths
// K_b = cu_q[b+1] - cu_q[b] - 1 (EMS-SD's samples with different numbers of
// prediction tokens, unpadded), else b*(K+1).
// One workgroup of 1024 threads per sequence; it computes its own scan offset,
// so the kernel needs no cross-workgroup synchronisation.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ int emitted(int n, int K) { return (n >= 0 && n <= K) ? n + 1 : 0; }

// First row and draft length of sequence b.
__device__ __forceinline__ int seq_q0(const CompactArgs& a, int b) {
    return a.cu_q ? a.cu_q[b] : b * (a.K + 1);
}
__device__ __forceinline__ int seq_k(const CompactArgs& a, int b) {
    return a.cu_q ? max(a.cu_q[b + 1] - a.cu_q[b] - 1, 0) : a.K;
}

// Copy `n16` 16-byte words of K and of V with every load of a batch issued
// before its stores: the copy takes one memory round trip per batch.  Indices
// past the end are clamped to the last word (re-read and re-written with its
// own value), so the batch needs no branches.
__device__ __forceinline__ void copy_rows16(const uint4* ks, const uint4* vs, uint4* kd, uint4* vd,
                                            size_t n16) {
    if (n16 == 0) return;
    const size_t last = n16 - 1;
    for (size_t base = threadIdx.x; base < n16; base += static_cast<size_t>(kThreads) * 4) {
        const size_t i0 = min(base, last), i1 = min(base + kThreads, last);
        const size_t i2 = min(base + 2 * kThreads, last), i3 = min(base + 3 * kThreads, last);
        const uint4 k0 = ks[i0], k1 = ks[i1], k2 = ks[i2], k3 = ks[i3];
        const uint4 v0 = vs[i0], v1 = vs[i1], v2 = vs[i2], v3 = vs[i3];
        kd[i0] = k0; kd[i1] = k1; kd[i2] = k2; kd[i3] = k3;
        vd[i0] = v0; vd[i1] = v1; vd[i2] = v2; vd[i3] = v3;
    }
}

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
    __shared__ int red[kThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x;
    // independent loads, issued together
    const int nb = a.n_accepted[b];
    const int L = a.kv_len[b];
    const int64_t start = a.kv_start[b];
    const int q0 = seq_q0(a, b);
    const int kb = seq_k(a, b);
    int part = 0;
    for (int i = tid; i < b; i += kThreads) part += emitted(a.n_accepted[i], seq_k(a, i));
    // the sequence's first 2048 output tokens (K_b + 1 of them are emitted at
    // most), loaded with the lengths rather than after the offset scan
    int tok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * kThreads;
        tok[u] = (i <= kb) ? a.out_tokens[static_cast<size_t>(q0) + i] : 0;
    }
    const int e = emitted(nb, kb);
    if (tid == 0 && e == 0) set_status(a.status, 4);

    const size_t row_bytes = static_cast<size_t>(a.Hkv) * a.D * a.elem_bytes;
    const size_t dst0 = static_cast<size_t>(start + L) * row_bytes;
    const size_t src0 = static_cast<size_t>(q0) * row_bytes;
    const size_t nbytes = static_cast<size_t>(e) * row_bytes;
    if (row_bytes % 16 == 0) {
        copy_rows16(reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src0),
                    reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src0),
                    reinterpret_cast<uint4*>(static_cast<char*>(a.k_cache) + dst0),
                    reinterpret_cast<uint4*>(static_cast<char*>(a.v_cache) + dst0), nbytes / 16);
    } else {
        const size_t n4 = nbytes / 4;
        for (size_t i = tid; i < 2 * n4; i += kThreads) {
            const bool v = i >= n4;
            const size_t k = v ? i - n4 : i;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(
                static_cast<const char*>(v ? a.v_new : a.k_new) + src0) + k;
            uint32_t* dst =
                reinterpret_cast<uint32_t*>(static_cast<char*>(v ? a.v_cache : a.k_cache) + dst0) + k;
            *dst = *src;
        }
    }
    const int cu = block_sum<kThreads>(part, red);  // also: every thread has read kv_len[b]
    if (tid == 0) {
        a.cu_tokens[b] = cu;
        if (b == a.B - 1) a.cu_tokens[a.B] = cu + e;
        a.kv_len[b] = L + e;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * kThreads;
        if (i < e) a.tokens_packed[cu + i] = tok[u];
    }
    for (int i = tid + 2 * kThreads; i < e; i += kThreads)  // draft lengths above 2047
        a.tokens_packed[cu + i] = a.out_tokens[static_cast<size_t>(q0) + i];
}

}  // namespace

hipError_t compact_launch(const CompactArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    hipLaunchKernelGGL(compact_kernel, dim3(a.B), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sv
