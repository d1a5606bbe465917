// Device image of a split-KV plan: the records the HIP kernels read.
//
// One image is built per plan on the host (plan.cpp) and copied to caller-owned
// device memory (splitkv_plan_upload). All offsets are byte offsets from the image
// base and are 16-byte aligned.
#pragma once
#include <stdint.h>

namespace splitkv {

// Per-sequence record.
struct SeqRec {
  int64_t kv_base;   // first token of the sequence in K / V
  int64_t q_base;    // first token of the sequence in Q / out / lse
  int64_t n;         // context length n_s
  int64_t row_base;  // first workspace row of the sequence
  int32_t q;         // trailing query count q_s
  int32_t nb;        // number of KV blocks, ceil(n_s / B)
  int32_t rows;      // query rows per KV head, q_s * g
  int32_t pad;
};
static_assert(sizeof(SeqRec) == 48, "SeqRec layout");

// One LPT unit: a context KV block of one sequence, for KV heads [kv0, kv0 + nkv).
struct UnitRec {
  int32_t seq;
  int32_t block;
  int32_t kv0;
  int32_t nkv;
};
static_assert(sizeof(UnitRec) == 16, "UnitRec layout");

// Keys per stage of the bf16 partial-attention pipeline, and the largest row count
// whose Q tile travels with a job's first stage. The planner uses both to cut units
// into jobs.
constexpr int32_t kStageKeys = 64;
constexpr int32_t kQTileRows = 64;
// Row tiles of 16 query rows that one pass of the bf16 kernel covers.
constexpr int32_t kPassTiles = 16;
// Passes of at least this many row tiles run on the matrix path (partial_mma.hip).
constexpr int32_t kMmaMinTiles = 8;

// Merged rows per merge workgroup (one wavefront each).
constexpr int32_t kMergeRowsPerGroup = 4;

// Where a merge workgroup's rows are: the index lo, in the merged sequence list, of the
// sequence holding the group's first row (row_base[lo] <= row < row_base[lo + 1]), with
// bit 31 set when a later row of the group lies in a later sequence, and that sequence's
// id s. One entry per workgroup, so a row finds its sequence in one load.
struct MergeGroup {
  int32_t lo_cross;
  int32_t seq;
};
static_assert(sizeof(MergeGroup) == 8, "MergeGroup layout");
constexpr int32_t kMergeCross = int32_t(0x80000000u);

// Keys per workgroup of the backward dK/dV kernel, and each such key tile's place: the
// sequence and the tile's index within it (tiles numbered sequence by sequence). The
// table lists the tiles of sequences with more than kFusedRows query rows per KV head;
// the others get their dK and dV in the pass that streams their blocks for dQ.
constexpr int32_t kDkvTileKeys = 64;
constexpr int32_t kFusedRows = 16;
struct KeyTile {
  int32_t seq;
  int32_t tile;
};
static_assert(sizeof(KeyTile) == 8, "KeyTile layout");

// The plan's scheduling area: kQueues uint32 counters of the shared tail's
// sub-queues (the next entry of each; one per 64-byte line, so that workgroups on
// different sub-queues do not contend), then the count of finished workgroups. Zero
// between launches.
constexpr int32_t kQueues = 8;
constexpr int32_t kSchedStride = 16;  // uint32 words between counters
constexpr uint64_t kSchedBytes = 1024;

// Job flags.
constexpr int32_t kJobWrMask = 3;   // log2 of the row groups the computing wavefronts form
constexpr int32_t kJobQTile = 4;    // Q rows of the job travel through LDS with stage 0
constexpr int32_t kJobSingle = 8;   // the sequence has a single block (its result is final)
constexpr int32_t kJobStream = 16;  // K/V read with the non-temporal hint (the block is not read again later)
constexpr int32_t kJobFusedKV = 32; // backward: the job holds all of its KV head's query rows (at most
                                    // kFusedRows), and its block's dK and dV come from the dQ pass

// One job of the bf16 partial-attention kernel: one pass over a block's keys for one
// KV head and up to kPassTiles row tiles of its query rows. Query row r of a KV head
// is query token i = r / g of the sequence, query head kv * g + r % g.
struct JobRec {
  int64_t kv_tok;   // token of the block's first key in K / V
  int64_t q_tok;    // token of the sequence's first query in Q / out / lse
  int64_t ws_row;   // workspace row of query row 0 for this (KV head, block)
  int32_t kv;       // KV head
  int32_t len;      // keys in the block
  int32_t lim0;     // causal: query token i sees block keys t <= lim0 + i
  int32_t rows;     // query rows of the KV head, q_s * g
  int32_t tile_lo;  // first row tile of this pass
  int32_t tile_n;   // row tiles in this pass
  int32_t nst;      // stages of kStageKeys keys that hold a visible key
  int32_t flags;    // kJob* bits
  int32_t pad[2];
};
static_assert(sizeof(JobRec) == 64, "JobRec layout");

// Offsets of the arrays inside the image.
struct ImageLayout {
  uint64_t seqs;        // SeqRec[S]
  uint64_t units;       // UnitRec[num_units], grouped by workgroup (the worker placed on it)
  uint64_t worker_ptr;  // int32[m + 1]: workgroup w runs units [worker_ptr[w], worker_ptr[w+1])
  uint64_t merge_all;   // int64[S + 1]: prefix of Hkv * rows over all sequences
  uint64_t merge_multi; // int32[S_multi] sequence ids with nb > 1, then
  uint64_t merge_multi_base;  // int64[S_multi + 1]: prefix of Hkv * rows over them
  uint64_t merge_groups_all;   // MergeGroup[ceil(rows / kMergeRowsPerGroup)] over all sequences
  uint64_t merge_groups_multi; // the same over the sequences with nb > 1
  uint64_t key_tiles;   // KeyTile[num_key_tiles]: the backward dK/dV kernel's key tiles
  uint64_t jobs;        // JobRec[num_jobs] in LPT order
  uint64_t wjobs;       // int32[num_jobs]: job indices of each workgroup's units, workgroup by workgroup
  uint64_t job_ptr;     // int32[m + 1]: workgroup w's jobs are wjobs[job_ptr[w] .. job_ptr[w+1])
  uint64_t split_ptr;   // int32[m]: of those, the matrix-path jobs come first, up to split_ptr[w]
  uint64_t chunk_ptr;   // int32[num_chunks + 1]: the shared tail's chunks of consecutive jobs
  uint64_t sched;       // kSchedBytes, 256-byte aligned: counters of the shared job queue
  uint64_t total;
};

}  // namespace splitkv
