// Host-side interface between the C ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- attention
struct AttnArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int64_t* kv_start;
    const int32_t* kv_len;
    const void* k_new;
    const void* v_new;
    const void* k_prefix;
    const void* v_prefix;
    void* out;
    int32_t* status;
    const int32_t* cu_q;  // ragged draft lengths: [B+1] device query-row offsets, or null
    int rows;             // query rows in all
    int B, K, Hq, Hkv, D, bf16, prefix_len;  // K: the largest draft length when ragged
    float scale;
    int chunk;          // keys per split-K work item of the per-sequence part
    int prefix_chunk;   // keys per work item of the shared prefix
    int slots;          // split-K work items per kv head (host upper bound)
    void* workspace;      // partial results (the data region of the plan)
    void* counters;       // arrival counters, zero on entry and left zero (null: at the
                          // start of `workspace`, which then holds the whole plan)
    hipEvent_t ev_start, ev_stop;  // optional records around the chunk kernel
};

// Sequences whose decode work plan travels in the kernel arguments.
constexpr int kAttnPlanB = 128;

// Chunking decisions made on the host from the host length bound.
struct AttnPlan {
    int chunk, prefix_chunk, slots, prefix_slots;
    int grid;    // bf16 path: workgroups (work items) of the decode kernel for the host bound
    int lambda;  // bf16 path: 16-key slices per work item at most
    int nct;     // bf16 path: 16-column tiles per work item (kernel instance)
    // bf16 path, B <= kAttnPlanB: chunk prefix sums, slices and first query
    // rows per sequence (plan_nb = B), else plan_nb = 0
    int plan_nb;
    int plan_q[kAttnPlanB + 1];
    int plan_s[kAttnPlanB];
    int plan_row0[kAttnPlanB + 1];
    // grouped heads (column waves): the 32-key items of all sequences cut into
    // plan_W equal ranges, each taken by Hkv workgroups, one per kv head
    // (plan_W = 0: per-sequence chunks); plan_s then counts 32-key items,
    // plan_q holds their prefix sums and plan_N all items
    int plan_W;
    long long plan_N;
    size_t bytes;          // whole workspace: counter region, then data region
    size_t counter_bytes;  // the counter region (B * Hkv arrival counters, 256-byte rounded)
    bool ok;  // false: the sequences are too long for the merge (unsupported)
};

// cu_q_host: [B+1] host query-row offsets of ragged draft lengths (K = their
// largest K_b), or null for K drafts in every sequence.
AttnPlan attn_plan(int B, int K, int Hq, int Hkv, int D, int bf16,
                   const int32_t* kv_len_host, const int32_t* cu_q_host, int prefix_len);
hipError_t attn_launch(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream);

// The library's fixed scratch array on the current device (allocation-free
// entry point): its counter region (zero between calls) and its data region.
// The first call on a device looks the array up and enqueues a clear of the
// counter region on `stream`.
hipError_t noalloc_scratch(hipStream_t stream, void** counters, size_t* counter_bytes,
                           void** data, size_t* data_bytes);
// The sizes of those two regions (no device call).
void noalloc_limits(size_t* counter_bytes, size_t* data_bytes);

// ---------------------------------------------------------------- sampler
struct AcceptArgs {
    const void* target_logits;
    const void* draft_logits;
    const int32_t* draft_tokens;
    const float* u_accept;
    const float* u_sample;
    int32_t* n_accepted;
    int32_t* out_tokens;
    int32_t* status;
    void* workspace;
    const int32_t* cu_q;  // ragged draft lengths: [B+1] device target-row offsets, or null
    int nt;               // target rows: cu_q[B], or B*(K+1)
    int B, K, V, bf16, greedy;  // K: the largest draft length when ragged
    float temperature, top_p;
    int top_k;            // keep the top_k largest logits (and ties) first; 0: off
    // the compaction fused into the call (spec_accept_compact); kv_len null: off
    int32_t* kv_len;
    const int64_t* kv_start;
    void* k_cache;
    void* v_cache;
    const void* k_new;
    const void* v_new;
    int32_t* tokens_packed;
    int32_t* cu_tokens;
    size_t row_bytes;     // Hkv * D * element size (a multiple of 4)
    // row statistics from the LM head (spec_accept_prestats); pre_m[0] null: none
    const float* pre_m[2];   // [0] target rows [nt][pre_parts], [1] draft rows
    const double* pre_s[2];
    int pre_parts;
};

// nt: target rows in all (B*(K+1) without ragged draft lengths)
size_t accept_workspace_bytes(int B, long long nt, int V);
int accept_max_vocab();
int accept_max_drafts();
hipError_t accept_launch(const AcceptArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- LM head
struct LmArgs {
    const void* hidden;   // [rows][H] bf16
    const void* weight;   // [V][H] bf16
    int rows, H, V;       // H a multiple of 32
    float temperature;
    float* logits;        // [rows][V] fp32
    float* part_max;      // [rows][lm_head_parts(V)]
    double* part_sum;
};
int lm_head_parts(int V);
int lm_head_part_len();
hipError_t lm_head_launch(const LmArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- compaction
struct CompactArgs {
    const int32_t* n_accepted;
    const int32_t* out_tokens;
    int32_t* kv_len;
    const int64_t* kv_start;
    void* k_cache;
    void* v_cache;
    const void* k_new;
    const void* v_new;
    int32_t* tokens_packed;
    int32_t* cu_tokens;
    int32_t* status;
    const int32_t* cu_q;  // ragged draft lengths: [B+1] device row offsets, or null
    int B, K, Hkv, D, elem_bytes;  // K: unused when ragged
};

hipError_t compact_launch(const CompactArgs& a, hipStream_t stream);

}  // namespace sv
