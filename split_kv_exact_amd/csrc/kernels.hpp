// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_image.hpp"

namespace splitkv {

// Arguments of the partial-attention kernels (one workgroup per LPT worker).
struct PartialArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;  // strides in elements
  float scale;                                 // softmax scale
  const SeqRec* seqs;
  const UnitRec* units;
  const int32_t* worker_ptr;
  const JobRec* jobs;       // bf16 kernel: jobs in LPT order
  const int32_t* wjobs;     // bf16 kernel: job indices of each worker's units
  const int32_t* job_ptr;   // bf16 kernels: workgroup w's jobs are wjobs[job_ptr[w] .. job_ptr[w+1]),
  const int32_t* split_ptr; //   the matrix-path jobs first, up to split_ptr[w]
  uint32_t* sched;          // bf16 kernel: queue counters (next chunk, workgroups done), zero between launches
  const int32_t* chunk_ptr; // bf16 kernel: the shared tail's chunks
  int32_t num_jobs;
  int32_t tail_start;       // bf16 kernel: jobs from here on come from the shared tail (num_jobs: none)
  int32_t num_chunks;
  int32_t queue;            // bf16 kernel: 1 = shared tail in use
  uint64_t* clock;          // null, or [2 * num_workers] start / end clocks per workgroup
  int32_t clock_add;        // bf16 kernel: an earlier launch wrote the clocks; add its busy time
  int32_t num_workers;
  int32_t Hq, Hkv, g, B, causal;
  float* ws_o;    // partial outputs [partial_rows, D] (fp32; fp16 elements when h16)
  float* ws_lse;  // partial LSEs [partial_rows] (fp32; (LSE, row scale) pairs when h16)
  // When non-null, sequences with a single block write their final result here
  // instead of the workspace (the fused path).
  float* out;
  float* lse;
  // Partials stored as fp16 elements times a per-row fp32 scale. Read on the host only:
  // the launch picks the kernel variant.
  int32_t h16;
};

// Arguments of the merge kernel (one wavefront per merged row).
struct MergeArgs {
  const SeqRec* seqs;
  const int32_t* seq_ids;    // sequences to merge (null: all sequences 0..count-1)
  const int64_t* row_base;   // prefix over those sequences of Hkv * rows
  const MergeGroup* groups;  // per workgroup: the sequence of its first row
  int32_t count;             // number of sequences to merge
  int64_t total_rows;        // row_base[count]
  int32_t Hq, Hkv, g;
  float scale;
  const float* ws_o;    // fp32 partial outputs, or fp16 elements when h16
  const float* ws_lse;  // fp32 LSEs, or (LSE, row scale) pairs when h16
  int32_t h16;
  float* out;
  float* lse;
};

// Arguments of the backward kernels (bf16 inputs; fp32 dQ, fp32 or bf16 dK and dV).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;                                    // dO, same dtype as q
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, do_st, do_sh;  // strides in elements
  float scale;
  const float* out;  // forward O [total_q, Hq, D], contiguous
  const float* lse;  // forward LSE [total_q, Hq]
  float* dq;         // [total_q, Hq, D], contiguous
  void* dk;          // [total_kv, Hkv, D], contiguous, fp32 or bf16 (dkv_bf16)
  void* dv;
  float* ws_dq;      // per (block, KV head) dQ parts [partial_rows, D]
  float* ws_d;       // D_i = <dO_i, O_i> [total_q * Hq]
  float* ws_l2;      // LSE_i * log2(e) [total_q * Hq], right after ws_d
  const SeqRec* seqs;
  int32_t S;
  const JobRec* jobs;
  int32_t num_jobs;
  int32_t num_fused_jobs;  // of which kJobFusedKV
  int32_t Hq, Hkv, g, causal;
  int64_t total_q;
  // Summing the dQ parts of multi-block sequences (the merge's row mapping).
  const int32_t* seq_ids;
  const int64_t* row_base;
  const MergeGroup* groups;
  int32_t count;
  int64_t total_rows;
  int64_t key_tiles;  // entries of the key-tile table (sequences of more than kFusedRows rows)
  const KeyTile* tiles;  // where each key tile lies
  int32_t dq_waves;   // waves per dQ workgroup: 4 when every pass has at most 8 row tiles, else 8
  int32_t dkv_bf16;   // dK and dV stored as bf16 (else fp32)
};

// Size of the library's own device workspace (splitkv_attn_scratch), one per GPU.
constexpr size_t kScratchBytes = size_t(256) << 20;

// Address of the calling thread's current device's copy of that workspace (looked up
// once per device with hipGetSymbolAddress, then cached).
hipError_t scratch_address(void** out);

hipError_t launch_partial_bf16(const PartialArgs& a, int head_dim, hipStream_t stream);
// partial_passes: some matrix-path pass has fewer than 16 row tiles.
hipError_t launch_partial_mma(const PartialArgs& a, int head_dim, bool partial_passes, hipStream_t stream);
hipError_t launch_backward_bf16(const BwdArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_partial_f32(const PartialArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream);

}  // namespace splitkv
