// pkv_kernels.hpp -- launch-side declarations shared by the kernel sources
// and the C ABI shim of libpagedkv.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// streaming-read probe (probe.hip)
hipError_t launch_stream_read(const void* buf, long long bytes, int waves, uint32_t* sink,
                              hipStream_t stream);

struct AppendArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    void* k_cache;
    void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int32_t max_blocks, B, Hkv, D, block_size, kv_dtype;   // kv_dtype: kernel format 0/1/2
    int32_t sc_blk, sc_head;
};

struct DecodeArgs {
    const uint16_t* query;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* out;           // single pass
    float* lse_out;       // single pass, may be null
    float* partial_out;   // split
    float* partial_lse;   // split
    const int32_t* query_start;  // several new tokens: [B + 1] row offsets, else null
    int32_t max_blocks, B, Hq, Hkv, G, split_tokens, max_splits;
    int32_t sc_blk, sc_head;     // scale of (block p, head h): k_scale[p * sc_blk + h * sc_head]
    int32_t total_rows;   // several new tokens: rows of query / out
    float scale_log2;     // softmax scale * log2(e)
    // Append fused into the decode launch: the step's new K/V rows
    // [B, Hkv, D] bf16, written (encoded like paged_kv_append) into slot
    // T_b - 1 of the caches above by the wave that attends that slot, before
    // it loads it; null: the caches are only read.
    const uint16_t* k_new = nullptr;
    const uint16_t* v_new = nullptr;
};

// The unit a work-group starts but leaves unfinished (b < 0: none), with
// everything its merge needs.
struct CutRecord {
    long long ustart;         // linear index of the unit's first tile
    long long total;          // tiles of the whole call
    long long rl;             // range holding the unit's last tile
    int32_t b, u;             // sequence, unit of the sequence in the tile list (head
                              // group of the list, column group)
    int32_t n, ncg;           // tiles of the unit, column groups of the sequence
    int32_t qs, q;            // several new tokens: first row and rows of the sequence
};

// Workspace of the balanced schedule: 2 partial slots per launched
// work-group, each with head_group * C rows (C = G for a decode step,
// 16 * column tiles with several new tokens) of D floats and as many lse,
// then one CutRecord per work-group.
struct BalanceArgs {
    float* part_out;          // [2 * ngroups_launched, head_group * C, D]
    float* part_lse;          // [2 * ngroups_launched, head_group * C]
    CutRecord* cuts;          // [ngroups_launched], 16-byte aligned
    int32_t ngroups_launched; // work-groups of the decode launch (a multiple of head_split)
    int32_t head_group;       // kv heads per work-group (divides Hkv, <= 8)
    int32_t head_split;       // work-groups sharing each token range (their head groups
                              // together cover head_group * head_split kv heads)
};

// Several new K/V rows per sequence: rows query_start[b] .. query_start[b+1]-1
// are positions T_b - q_b .. T_b - 1 of sequence b.
struct WriteArgs {
    const uint16_t* k_rows;
    const uint16_t* v_rows;
    const int32_t* query_start;
    void* k_cache;
    void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int32_t max_blocks, B, max_query_len, Hkv, D, block_size, kv_dtype;   // format 0/1/2
    int32_t sc_blk, sc_head;
};

// Whole-block moves: destination block dst_ids[i] (i if null) of the
// destination pools takes source block src_ids[i] (i if null).
struct BlockMoveArgs {
    const unsigned char* src_k;
    const unsigned char* src_v;
    unsigned char* dst_k;
    unsigned char* dst_v;
    const float* src_ks;      // fp8 scales [.., scale_count], or null
    const float* src_vs;
    float* dst_ks;
    float* dst_vs;
    const int32_t* src_ids;
    const int32_t* dst_ids;
    long long block_bytes;    // bytes of one K (or V) block, a multiple of 16
    int32_t n;                // blocks to move
    int32_t scale_count;      // scales per block (Hkv) when fp8, else 0
};

struct ReduceArgs {
    const float* partial_out;
    const float* partial_lse;
    const int32_t* context_lens;
    float* out;
    float* lse_out;
    int32_t B, Hq, D, split_tokens, max_splits;
};

// Kernel formats: the C ABI's kv_dtype codes map to 0 (bf16), 1 (E4M3FN,
// any scale granularity) or 2 (uint8 with zero point); the scale of block p,
// kv head h is at [p * sc_blk + h * sc_head] (its zero point at + 1).
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// nt: stream the K/V loads with the non-temporal hint
hipError_t launch_decode(const DecodeArgs& a, int D, int block_size, int kv_dtype, bool nt,
                         hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_decode_balanced(const DecodeArgs& a, const BalanceArgs& ws, int D,
                                  int block_size, int kv_dtype, bool nt, hipStream_t stream);
hipError_t launch_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_move_blocks(const BlockMoveArgs& a, hipStream_t stream);
// Causal attention of several new tokens per sequence on the balanced
// schedule; nct = 16-column MFMA tiles per wave (1 or 2).
hipError_t launch_multiquery(const DecodeArgs& a, const BalanceArgs& ws, int D, int block_size,
                             int kv_dtype, int nct, bool nt, hipStream_t stream);
// Long runs of new tokens: one work-group per 256 (row, head) columns of a
// (sequence, kv head), K/V tiles shared through LDS; no workspace.
hipError_t launch_prefill(const DecodeArgs& a, int max_query_len, int D, int block_size,
                          int kvf, bool nt, hipStream_t stream);
// resident work-groups per compute unit of the multi-query kernel (0 on error)
int multiquery_groups_per_cu(int D, int block_size, int kv_dtype, int head_group, int nct);
// kv heads per work-group of the balanced schedule for Hkv kv heads
// (nct = 0: decode; 1 or 2: the multi-query kernel's column tiles; kvf:
// kernel format 0/1/2)
int balanced_head_group(int Hkv, int nct, int kvf);
// whether that schedule launches one work-group per CU (else as many as fit)
bool balanced_one_group_per_cu(int Hkv, int nct, int kvf);
// resident work-groups per compute unit of the balanced decode (0 on error)
int balanced_groups_per_cu(int D, int block_size, int kv_dtype, int head_group);

} // namespace pkv
