// C ABI of libsplitkv: argument checks, plan handling and kernel dispatch.
//
// Every argument check happens before any HIP call, so malformed calls fail the same
// way with or without a GPU. The library allocates no device memory and never
// synchronises a stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "kernels.hpp"
#include "plan.hpp"
#include "splitkv.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_plan(const splitkv_plan_t* pl, const void* dev_plan) {
  if (!pl) return fail(SPLITKV_ERR_INVALID_ARG, "plan is NULL");
  if (!dev_plan) return fail(SPLITKV_ERR_INVALID_ARG, "dev_plan is NULL");
  if (!aligned16(dev_plan)) return fail(SPLITKV_ERR_INVALID_ARG, "dev_plan must be 16-byte aligned");
  return SPLITKV_OK;
}

int check_inputs(const splitkv_plan_t* pl, const splitkv_inputs* in, float* scale_out) {
  if (!in) return fail(SPLITKV_ERR_INVALID_ARG, "inputs is NULL");
  if (in->dtype != SPLITKV_F32 && in->dtype != SPLITKV_BF16) return fail(SPLITKV_ERR_INVALID_ARG, "unknown dtype");
  if (in->dtype == SPLITKV_F32 && pl->pfmt == SPLITKV_PARTIAL_F16_ROWSCALE)
    return fail(SPLITKV_ERR_UNSUPPORTED, "fp32 inputs need a plan with fp32 partials (partial_format 0)");
  if (pl->D != 64 && pl->D != 128)
    return fail(SPLITKV_ERR_UNSUPPORTED, "kernels exist for head_dim 64 and 128 only");
  if (!in->q || !in->k || !in->v) return fail(SPLITKV_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  if (!aligned16(in->q) || !aligned16(in->k) || !aligned16(in->v))
    return fail(SPLITKV_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  const int64_t vec = in->dtype == SPLITKV_F32 ? 4 : 8;  // elements per 16 bytes
  const int64_t st[6] = {in->q_stride_tok, in->q_stride_head, in->k_stride_tok,
                         in->k_stride_head, in->v_stride_tok, in->v_stride_head};
  for (int64_t x : st)
    if (x < 0 || x % vec != 0)
      return fail(SPLITKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  if (in->schedule != SPLITKV_SCHED_AUTO && in->schedule != SPLITKV_SCHED_QUEUE &&
      in->schedule != SPLITKV_SCHED_STATIC)
    return fail(SPLITKV_ERR_INVALID_ARG, "unknown schedule");
  if ((reinterpret_cast<uintptr_t>(in->worker_clock) & 7u) != 0)
    return fail(SPLITKV_ERR_INVALID_ARG, "worker_clock must be 8-byte aligned");
  // The bf16 kernel addresses a lane's rows within one stage or Q tile with 32-bit
  // byte offsets.
  if (in->dtype == SPLITKV_BF16)
    for (int64_t x : st)
      if (x > (int64_t(1) << 24))
        return fail(SPLITKV_ERR_UNSUPPORTED, "bf16 strides must be at most 2^24 elements");
  if (!(std::isfinite(in->scale)) || in->scale < 0.f)
    return fail(SPLITKV_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  *scale_out = in->scale == 0.f ? float(1.0 / std::sqrt(double(pl->D))) : in->scale;
  return SPLITKV_OK;
}

int check_ws(const splitkv_plan_t* pl, const void* ws, size_t ws_bytes) {
  if (!ws) return fail(SPLITKV_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(SPLITKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < pl->ws_bytes)
    return fail(SPLITKV_ERR_WORKSPACE, "workspace needs " + std::to_string(pl->ws_bytes) + " bytes, got " +
                                           std::to_string(ws_bytes));
  return SPLITKV_OK;
}

int check_out(const float* out, const float* lse) {
  if (!out || !lse) return fail(SPLITKV_ERR_INVALID_ARG, "out and lse must be non-NULL");
  if (!aligned16(out)) return fail(SPLITKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(SPLITKV_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return SPLITKV_OK;
}

splitkv::PartialArgs partial_args(const splitkv_plan_t* pl, void* dev_plan, const splitkv_inputs* in,
                                  float scale, float* ws) {
  const uint8_t* base = static_cast<const uint8_t*>(dev_plan);
  splitkv::PartialArgs a{};
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.q_st = in->q_stride_tok;
  a.q_sh = in->q_stride_head;
  a.k_st = in->k_stride_tok;
  a.k_sh = in->k_stride_head;
  a.v_st = in->v_stride_tok;
  a.v_sh = in->v_stride_head;
  a.scale = scale;
  a.seqs = reinterpret_cast<const splitkv::SeqRec*>(base + pl->layout.seqs);
  a.units = reinterpret_cast<const splitkv::UnitRec*>(base + pl->layout.units);
  a.worker_ptr = reinterpret_cast<const int32_t*>(base + pl->layout.worker_ptr);
  a.jobs = reinterpret_cast<const splitkv::JobRec*>(base + pl->layout.jobs);
  a.wjobs = reinterpret_cast<const int32_t*>(base + pl->layout.wjobs);
  a.job_ptr = reinterpret_cast<const int32_t*>(base + pl->layout.job_ptr);
  a.split_ptr = reinterpret_cast<const int32_t*>(base + pl->layout.split_ptr);
  a.sched = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(dev_plan) + pl->layout.sched);
  a.chunk_ptr = reinterpret_cast<const int32_t*>(base + pl->layout.chunk_ptr);
  a.num_jobs = int32_t(pl->num_jobs);
  const bool queue = in->schedule == SPLITKV_SCHED_QUEUE || (in->schedule == SPLITKV_SCHED_AUTO && pl->queue_default);
  a.queue = queue && pl->tail_start < pl->num_jobs ? 1 : 0;
  a.tail_start = a.queue ? pl->tail_start : a.num_jobs;
  a.num_chunks = int32_t(pl->chunk_ptr.size()) - 1;
  a.clock = in->worker_clock;
  a.num_workers = pl->m;
  a.Hq = pl->Hq;
  a.Hkv = pl->Hkv;
  a.g = pl->g;
  a.B = pl->B;
  a.causal = pl->causal;
  a.ws_o = ws;
  a.ws_lse = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pl->ws_lse_offset);
  a.h16 = pl->pfmt == SPLITKV_PARTIAL_F16_ROWSCALE ? 1 : 0;
  a.out = nullptr;
  a.lse = nullptr;
  return a;
}

splitkv::MergeArgs merge_args(const splitkv_plan_t* pl, const void* dev_plan, const float* ws, float* out, float* lse,
                              bool multi_only) {
  const uint8_t* base = static_cast<const uint8_t*>(dev_plan);
  splitkv::MergeArgs m{};
  m.seqs = reinterpret_cast<const splitkv::SeqRec*>(base + pl->layout.seqs);
  if (multi_only) {
    m.seq_ids = reinterpret_cast<const int32_t*>(base + pl->layout.merge_multi);
    m.row_base = reinterpret_cast<const int64_t*>(base + pl->layout.merge_multi_base);
    m.groups = reinterpret_cast<const splitkv::MergeGroup*>(base + pl->layout.merge_groups_multi);
    m.count = pl->num_multi;
    m.total_rows = pl->merge_rows_multi;
  } else {
    m.seq_ids = nullptr;
    m.row_base = reinterpret_cast<const int64_t*>(base + pl->layout.merge_all);
    m.groups = reinterpret_cast<const splitkv::MergeGroup*>(base + pl->layout.merge_groups_all);
    m.count = pl->S;
    m.total_rows = pl->merge_rows_all;
  }
  m.Hq = pl->Hq;
  m.Hkv = pl->Hkv;
  m.g = pl->g;
  m.ws_o = ws;
  m.ws_lse = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ws) + pl->ws_lse_offset);
  m.h16 = pl->pfmt == SPLITKV_PARTIAL_F16_ROWSCALE ? 1 : 0;
  m.out = out;
  m.lse = lse;
  return m;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SPLITKV_OK;
  return fail(SPLITKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// bf16: the matrix-path jobs (passes of at least 8 row tiles) in one launch, then the
// other jobs in a second launch on the same stream; each launch only when it has jobs.
int launch_partial(const splitkv_plan_t* pl, splitkv::PartialArgs a, int dtype, hipStream_t stream) {
  if (dtype != SPLITKV_BF16) return hip_status(splitkv::launch_partial_f32(a, pl->D, stream), "partial attention launch");
  const bool mma = pl->num_mma_jobs > 0, rest = pl->num_jobs > pl->num_mma_jobs;
  if (mma)
    if (int st = hip_status(splitkv::launch_partial_mma(a, pl->D, pl->mma_partial_passes, stream),
                            "partial attention launch"))
      return st;
  a.clock_add = mma ? 1 : 0;
  if (rest || !mma) return hip_status(splitkv::launch_partial_bf16(a, pl->D, stream), "partial attention launch");
  return SPLITKV_OK;
}

}  // namespace

extern "C" {

int splitkv_version(void) { return (SPLITKV_VERSION_MAJOR << 16) | SPLITKV_VERSION_MINOR; }

int splitkv_plan(const splitkv_problem* problem, splitkv_plan_t** out) {
  g_last_error.clear();
  if (!out) return fail(SPLITKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  std::string why;
  if (!splitkv::validate_problem(problem, &why)) return fail(SPLITKV_ERR_INVALID_ARG, why);
  splitkv_plan_t* pl = nullptr;
  try {
    pl = new splitkv_plan_t();
    splitkv::build_plan(problem, pl);
  } catch (const std::bad_alloc&) {
    delete pl;
    return fail(SPLITKV_ERR_ALLOC, "host allocation failed while planning");
  }
  *out = pl;
  return SPLITKV_OK;
}

int splitkv_plan_info_get(const splitkv_plan_t* pl, splitkv_plan_info* info) {
  g_last_error.clear();
  if (!pl || !info) return fail(SPLITKV_ERR_INVALID_ARG, "plan and info must be non-NULL");
  info->num_units = int64_t(pl->u_cost.size());
  info->total_cost = pl->total_cost;
  info->makespan = pl->makespan;
  info->lower_bound = pl->lower_bound;
  info->imbalance = pl->imbalance;
  info->total_q = pl->total_q;
  info->total_kv = pl->total_kv;
  info->partial_rows = pl->partial_rows;
  info->plan_bytes = pl->image.size();
  info->workspace_bytes = pl->ws_bytes;
  info->ws_lse_offset = pl->ws_lse_offset;
  info->num_jobs = pl->num_jobs;
  info->exec_imbalance_static = pl->exec_static;
  info->exec_imbalance_static_est = pl->exec_static_est;
  info->exec_imbalance_queue_est = pl->exec_queue_est;
  info->auto_schedule = pl->queue_default && pl->tail_start < pl->num_jobs ? SPLITKV_SCHED_QUEUE : SPLITKV_SCHED_STATIC;
  info->num_mma_jobs = pl->num_mma_jobs;
  info->mma_partial_passes = pl->num_mma_jobs > 0 && pl->mma_partial_passes ? 1 : 0;
  info->partial_format = pl->pfmt;
  return SPLITKV_OK;
}

int splitkv_plan_export(const splitkv_plan_t* pl, int32_t* unit_seq, int32_t* unit_block, int32_t* unit_kv_head,
                        int32_t* unit_len, int64_t* unit_cost, int32_t* worker_of, int32_t* worker_ptr,
                        int32_t* worker_units, int64_t* load) {
  g_last_error.clear();
  if (!pl) return fail(SPLITKV_ERR_INVALID_ARG, "plan is NULL");
  const size_t n = pl->u_cost.size();
  if (unit_seq) std::memcpy(unit_seq, pl->u_seq.data(), n * sizeof(int32_t));
  if (unit_block) std::memcpy(unit_block, pl->u_block.data(), n * sizeof(int32_t));
  if (unit_kv_head) std::memcpy(unit_kv_head, pl->u_kv.data(), n * sizeof(int32_t));
  if (unit_len) std::memcpy(unit_len, pl->u_len.data(), n * sizeof(int32_t));
  if (unit_cost) std::memcpy(unit_cost, pl->u_cost.data(), n * sizeof(int64_t));
  if (worker_of) std::memcpy(worker_of, pl->worker_of.data(), n * sizeof(int32_t));
  if (worker_ptr) std::memcpy(worker_ptr, pl->worker_ptr.data(), pl->worker_ptr.size() * sizeof(int32_t));
  if (worker_units) std::memcpy(worker_units, pl->worker_units.data(), n * sizeof(int32_t));
  if (load) std::memcpy(load, pl->load.data(), pl->load.size() * sizeof(int64_t));
  return SPLITKV_OK;
}

int splitkv_plan_upload(const splitkv_plan_t* pl, void* dev_plan, size_t bytes, void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  if (bytes < pl->image.size())
    return fail(SPLITKV_ERR_WORKSPACE, "plan buffer needs " + std::to_string(pl->image.size()) + " bytes");
  return hip_status(hipMemcpyAsync(dev_plan, pl->image.data(), pl->image.size(), hipMemcpyHostToDevice,
                                   static_cast<hipStream_t>(hip_stream)),
                    "plan upload");
}

void splitkv_plan_destroy(splitkv_plan_t* pl) { delete pl; }

int splitkv_partial_attn(const splitkv_plan_t* pl, void* dev_plan, const splitkv_inputs* in, float* ws,
                         size_t ws_bytes, void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  float scale = 0.f;
  if (int st = check_inputs(pl, in, &scale)) return st;
  if (int st = check_ws(pl, ws, ws_bytes)) return st;
  const splitkv::PartialArgs a = partial_args(pl, dev_plan, in, scale, ws);
  return launch_partial(pl, a, in->dtype, static_cast<hipStream_t>(hip_stream));
}

int splitkv_merge(const splitkv_plan_t* pl, const void* dev_plan, const float* ws, size_t ws_bytes, float* out,
                  float* lse, void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  if (pl->D != 64 && pl->D != 128)
    return fail(SPLITKV_ERR_UNSUPPORTED, "kernels exist for head_dim 64 and 128 only");
  if (int st = check_ws(pl, ws, ws_bytes)) return st;
  if (int st = check_out(out, lse)) return st;
  const splitkv::MergeArgs m = merge_args(pl, dev_plan, ws, out, lse, false);
  return hip_status(splitkv::launch_merge(m, pl->D, static_cast<hipStream_t>(hip_stream)), "merge launch");
}

int splitkv_attn(const splitkv_plan_t* pl, void* dev_plan, const splitkv_inputs* in, float* ws, size_t ws_bytes,
                 float* out, float* lse, void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  float scale = 0.f;
  if (int st = check_inputs(pl, in, &scale)) return st;
  if (int st = check_ws(pl, ws, ws_bytes)) return st;
  if (int st = check_out(out, lse)) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  splitkv::PartialArgs a = partial_args(pl, dev_plan, in, scale, ws);
  a.out = out;
  a.lse = lse;
  if (int st = launch_partial(pl, a, in->dtype, stream)) return st;
  const splitkv::MergeArgs m = merge_args(pl, dev_plan, ws, out, lse, true);
  return hip_status(splitkv::launch_merge(m, pl->D, stream), "merge launch");
}

int splitkv_attn_scratch(const splitkv_plan_t* pl, void* dev_plan, const splitkv_inputs* in, float* out, float* lse,
                         void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  float scale = 0.f;
  if (int st = check_inputs(pl, in, &scale)) return st;
  if (int st = check_out(out, lse)) return st;
  if (pl->ws_bytes > splitkv::kScratchBytes)
    return fail(SPLITKV_ERR_WORKSPACE, "the plan needs a workspace of " + std::to_string(pl->ws_bytes) +
                                           " bytes; the library's own holds " +
                                           std::to_string(splitkv::kScratchBytes) + " (use splitkv_attn)");
  void* ws = nullptr;
  if (int st = hip_status(splitkv::scratch_address(&ws), "scratch workspace address")) return st;
  return splitkv_attn(pl, dev_plan, in, static_cast<float*>(ws), splitkv::kScratchBytes, out, lse, hip_stream);
}

int splitkv_attn_backward(const splitkv_plan_t* pl, const void* dev_plan, const splitkv_inputs* in,
                          const splitkv_grads* gr, float* ws, size_t ws_bytes, void* hip_stream) {
  g_last_error.clear();
  if (int st = check_plan(pl, dev_plan)) return st;
  float scale = 0.f;
  if (int st = check_inputs(pl, in, &scale)) return st;
  if (in->dtype != SPLITKV_BF16) return fail(SPLITKV_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs only");
  if (!gr) return fail(SPLITKV_ERR_INVALID_ARG, "grads is NULL");
  if (!gr->d_out || !gr->out || !gr->lse || !gr->dq || !gr->dk || !gr->dv)
    return fail(SPLITKV_ERR_INVALID_ARG, "d_out, out, lse, dq, dk and dv must be non-NULL");
  if (!aligned16(gr->d_out) || !aligned16(gr->out) || !aligned16(gr->dq) || !aligned16(gr->dk) ||
      !aligned16(gr->dv))
    return fail(SPLITKV_ERR_INVALID_ARG, "d_out, out, dq, dk and dv must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(gr->lse) & 3u) != 0) return fail(SPLITKV_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (gr->dkv_dtype != SPLITKV_F32 && gr->dkv_dtype != SPLITKV_BF16)
    return fail(SPLITKV_ERR_INVALID_ARG, "dkv_dtype must be SPLITKV_F32 or SPLITKV_BF16");
  for (int64_t x : {gr->do_stride_tok, gr->do_stride_head}) {
    if (x < 0 || x % 8 != 0) return fail(SPLITKV_ERR_INVALID_ARG, "d_out strides must be non-negative multiples of 16 bytes");
    if (x > (int64_t(1) << 24)) return fail(SPLITKV_ERR_UNSUPPORTED, "bf16 strides must be at most 2^24 elements");
  }
  if (int st = check_ws(pl, ws, ws_bytes)) return st;
  const uint8_t* base = static_cast<const uint8_t*>(dev_plan);
  splitkv::BwdArgs b{};
  b.q = in->q;
  b.k = in->k;
  b.v = in->v;
  b.dout = gr->d_out;
  b.q_st = in->q_stride_tok;
  b.q_sh = in->q_stride_head;
  b.k_st = in->k_stride_tok;
  b.k_sh = in->k_stride_head;
  b.v_st = in->v_stride_tok;
  b.v_sh = in->v_stride_head;
  b.do_st = gr->do_stride_tok;
  b.do_sh = gr->do_stride_head;
  b.scale = scale;
  b.out = gr->out;
  b.lse = gr->lse;
  b.dq = gr->dq;
  b.dk = gr->dk;
  b.dv = gr->dv;
  b.ws_dq = ws;
  b.ws_d = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pl->ws_lse_offset);
  b.ws_l2 = b.ws_d + pl->total_q * pl->Hq;
  b.seqs = reinterpret_cast<const splitkv::SeqRec*>(base + pl->layout.seqs);
  b.S = pl->S;
  b.jobs = reinterpret_cast<const splitkv::JobRec*>(base + pl->layout.jobs);
  b.num_jobs = int32_t(pl->num_jobs);
  b.num_fused_jobs = int32_t(pl->num_fused_jobs);
  b.Hq = pl->Hq;
  b.Hkv = pl->Hkv;
  b.g = pl->g;
  b.causal = pl->causal;
  b.total_q = pl->total_q;
  b.seq_ids = reinterpret_cast<const int32_t*>(base + pl->layout.merge_multi);
  b.row_base = reinterpret_cast<const int64_t*>(base + pl->layout.merge_multi_base);
  b.groups = reinterpret_cast<const splitkv::MergeGroup*>(base + pl->layout.merge_groups_multi);
  b.count = pl->num_multi;
  b.total_rows = pl->merge_rows_multi;
  b.key_tiles = pl->num_key_tiles;
  b.tiles = reinterpret_cast<const splitkv::KeyTile*>(base + pl->layout.key_tiles);
  b.dq_waves = pl->max_rows <= 128 ? 4 : 8;
  b.dkv_bf16 = gr->dkv_dtype == SPLITKV_BF16;
  return hip_status(splitkv::launch_backward_bf16(b, pl->D, static_cast<hipStream_t>(hip_stream)),
                    "backward launch");
}

const char* splitkv_status_string(int status) {
  switch (status) {
    case SPLITKV_OK: return "ok";
    case SPLITKV_ERR_INVALID_ARG: return "invalid argument";
    case SPLITKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPLITKV_ERR_WORKSPACE: return "buffer too small";
    case SPLITKV_ERR_HIP: return "HIP runtime error";
    case SPLITKV_ERR_ALLOC: return "host allocation failed";
    default: return "unknown status";
  }
}

const char* splitkv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
