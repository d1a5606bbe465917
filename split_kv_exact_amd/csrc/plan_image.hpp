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

// Offsets of the arrays inside the image.
struct ImageLayout {
  uint64_t seqs;        // SeqRec[S]
  uint64_t units;       // UnitRec[num_units], grouped by worker (worker order)
  uint64_t worker_ptr;  // int32[m + 1]: worker w owns units [worker_ptr[w], worker_ptr[w+1])
  uint64_t merge_all;   // int64[S + 1]: prefix of Hkv * rows over all sequences
  uint64_t merge_multi; // int32[S_multi] sequence ids with nb > 1, then
  uint64_t merge_multi_base;  // int64[S_multi + 1]: prefix of Hkv * rows over them
  uint64_t total;
};

}  // namespace splitkv
