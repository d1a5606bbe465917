// Host-side LPT planner for split-KV attention (no HIP calls).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "plan_image.hpp"
#include "splitkv.h"

struct splitkv_plan_s {
  // Problem.
  int32_t S = 0, Hq = 0, Hkv = 0, D = 0, B = 0, m = 0, causal = 0, granularity = 0, g = 0;
  int32_t ridge = 0;  // cost_ridge_rows of the problem
  int32_t pfmt = 0;   // partial_format of the problem (splitkv_partial_format)
  std::vector<int32_t> xcd_speed;    // [8] relative speeds, or empty
  std::vector<int32_t> slot_worker;  // the plan worker run by workgroup s
  std::vector<int64_t> kv_lens;
  std::vector<int32_t> q_lens;

  // Units in enumeration order (seq, block, kv head).
  std::vector<int32_t> u_seq, u_block, u_kv, u_len;
  std::vector<int64_t> u_cost;

  // Assignment.
  std::vector<int32_t> worker_of, worker_ptr, worker_units;
  std::vector<int64_t> load;
  int64_t total_cost = 0, makespan = 0, lower_bound = 0;
  double imbalance = 0.0;

  // Layout.
  std::vector<splitkv::SeqRec> seqs;
  int64_t total_q = 0, total_kv = 0, partial_rows = 0;
  int64_t merge_rows_all = 0, merge_rows_multi = 0;
  int32_t num_multi = 0;  // sequences with more than one block
  int64_t num_key_tiles = 0;  // sum of ceil(n_s / kDkvTileKeys) over sequences of more than kFusedRows rows
  int32_t max_rows = 0;   // max_s q_s * g
  int64_t num_jobs = 0;   // jobs of the bf16 kernels
  int64_t num_fused_jobs = 0;  // of which flagged kJobFusedKV (backward: dK/dV from the dQ pass)
  int64_t num_mma_jobs = 0;  // of which the matrix-path launch runs the first num_mma_jobs
  bool mma_partial_passes = false;  // some matrix-path job has fewer than kPassTiles row tiles
  int32_t tail_start = 0;  // queue schedule: first job of the shared tail
  bool queue_default = false;  // SPLITKV_SCHED_AUTO picks the queue
  std::vector<int32_t> chunk_ptr;  // queue schedule: chunk c is jobs [chunk_ptr[c], chunk_ptr[c+1])
  // Modelled imbalance, (m * max - total) / total over the workgroups, of the schedules
  // as they run: the static lists under the page's cost and under the job-time
  // estimate, and the queue schedule simulated with that estimate.
  double exec_static = 0.0, exec_static_est = 0.0, exec_queue_est = 0.0;
  size_t ws_bytes = 0, ws_lse_offset = 0;

  // Device image.
  splitkv::ImageLayout layout{};
  std::vector<uint8_t> image;
};

namespace splitkv {

// Validate a problem; on failure returns false and sets *why.
bool validate_problem(const splitkv_problem* p, std::string* why);

// Build a plan (problem already validated). Throws std::bad_alloc on allocation failure.
void build_plan(const splitkv_problem* p, splitkv_plan_t* pl);

}  // namespace splitkv
