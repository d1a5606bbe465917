// Cost-aware LPT placement of context KV blocks on workers (host code only).
//
// Split-KV page, "Timeline": context KV blocks are allocated by a cost-aware
// longest-processing-time-first strategy with a reported load imbalance below 1%.
// The page gives no cost model, tie-break or imbalance definition; this planner uses
//   unit       = (sequence, block, KV head), enumerated in that order (or a whole
//                (sequence, block) serving every query head: the coarse granularity);
//   cost       = q_s * block length * query heads served (exact int64), or with a
//                ridge R > 0 the roofline-aware len * max(q_s * g, R) per KV head;
//   order      = costs descending, ties in enumeration order (stable sort);
//   placement  = worker with the smallest (load, index) via a binary min-heap;
//   imbalance  = (m * max_load - total) / total, one float64 division.
// With these rules the plan is unique, so it can be compared bit for bit.
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <functional>
#include <numeric>
#include <queue>
#include <utility>

namespace splitkv {

static inline uint64_t align16(uint64_t x) { return (x + 15) & ~uint64_t(15); }

bool validate_problem(const splitkv_problem* p, std::string* why) {
  auto fail = [&](const char* msg) {
    *why = msg;
    return false;
  };
  if (!p) return fail("problem is NULL");
  if (p->batch < 1) return fail("batch must be >= 1");
  if (!p->kv_lens || !p->q_lens) return fail("kv_lens and q_lens must be non-NULL");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1) return fail("head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0) return fail("num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim < 1) return fail("head_dim must be >= 1");
  if (p->block_len < 1 || p->block_len > (1 << 30)) return fail("block_len must be in [1, 2^30]");
  if (p->num_workers < 1) return fail("num_workers must be >= 1");
  if (p->causal != 0 && p->causal != 1) return fail("causal must be 0 or 1");
  if (p->granularity != SPLITKV_UNIT_SEQ_BLOCK_KVHEAD && p->granularity != SPLITKV_UNIT_SEQ_BLOCK)
    return fail("unknown granularity");
  if (p->cost_ridge_rows < 0 || p->cost_ridge_rows > (1 << 30)) return fail("cost_ridge_rows must be in [0, 2^30]");
  if (p->partial_format != SPLITKV_PARTIAL_F32 && p->partial_format != SPLITKV_PARTIAL_F16_ROWSCALE)
    return fail("unknown partial_format");
  if (p->xcd_speed)
    for (int x = 0; x < 8; ++x)
      if (p->xcd_speed[x] < 1) return fail("xcd_speed entries must be >= 1");
  const int64_t g = p->num_q_heads / p->num_kv_heads;
  for (int32_t s = 0; s < p->batch; ++s) {
    if (p->q_lens[s] < 1) return fail("every q_len must be >= 1");
    if (p->kv_lens[s] < p->q_lens[s]) return fail("every kv_len must be >= its q_len");
    if (p->kv_lens[s] > (int64_t(1) << 40)) return fail("kv_len too large");
    // Keep per-unit row counts in int32 and per-unit costs far from int64 overflow.
    if (int64_t(p->q_lens[s]) * g > (int64_t(1) << 30)) return fail("q_len * group too large");
  }
  // Every unit cost and their sum must stay exact in int64: bound the sum, per
  // sequence len * max(q * g, R) * Hkv over its n_s keys, in floating point.
  double total = 0.0;
  for (int32_t s = 0; s < p->batch; ++s)
    total += double(p->kv_lens[s]) * double(std::max<int64_t>(int64_t(p->q_lens[s]) * g, p->cost_ridge_rows)) *
             double(p->num_kv_heads);
  if (total > 4.0e18) return fail("total unit cost beyond 2^62");
  // Block, unit, job and token indices are int32 in the plan records and the kernels:
  // the block count of a sequence, the number of units and the number of jobs (a unit
  // per KV head and pass of up to kPassTiles row tiles) must fit, and so must the number
  // of kDkvTileKeys-key tiles the backward pass numbers.
  const int64_t imax = INT32_MAX;
  int64_t units = 0, jobs = 0, key_tiles = 0;
  for (int32_t s = 0; s < p->batch; ++s) {
    const int64_t nb = (p->kv_lens[s] + p->block_len - 1) / p->block_len;
    if (nb > imax) return fail("a sequence has more than 2^31 - 1 blocks");
    const int64_t tiles = (int64_t(p->q_lens[s]) * g + 15) / 16;
    const int64_t passes = (tiles + kPassTiles - 1) / kPassTiles;
    const int64_t per_block = p->granularity == SPLITKV_UNIT_SEQ_BLOCK_KVHEAD ? p->num_kv_heads : 1;
    units += nb * per_block;
    jobs += nb * p->num_kv_heads * passes;
    key_tiles += (p->kv_lens[s] + kDkvTileKeys - 1) / kDkvTileKeys;
    if (units > imax || jobs > imax) return fail("more than 2^31 - 1 units or jobs");
    if (key_tiles > imax) return fail("more than 2^31 - 1 key tiles of the backward pass");
  }
  return true;
}

void build_plan(const splitkv_problem* p, splitkv_plan_t* pl) {
  pl->S = p->batch;
  pl->Hq = p->num_q_heads;
  pl->Hkv = p->num_kv_heads;
  pl->D = p->head_dim;
  pl->B = p->block_len;
  pl->m = p->num_workers;
  pl->causal = p->causal;
  pl->granularity = p->granularity;
  pl->ridge = p->cost_ridge_rows;
  pl->pfmt = p->partial_format;
  pl->xcd_speed.clear();
  if (p->xcd_speed) pl->xcd_speed.assign(p->xcd_speed, p->xcd_speed + 8);
  pl->g = p->num_q_heads / p->num_kv_heads;
  pl->kv_lens.assign(p->kv_lens, p->kv_lens + p->batch);
  pl->q_lens.assign(p->q_lens, p->q_lens + p->batch);

  const int32_t S = pl->S, Hkv = pl->Hkv, g = pl->g, B = pl->B, m = pl->m;
  const bool per_head = pl->granularity == SPLITKV_UNIT_SEQ_BLOCK_KVHEAD;
  const int64_t heads = per_head ? g : pl->Hq;

  // Sequence records and workspace layout.
  pl->seqs.resize(S);
  int64_t kv_base = 0, q_base = 0, row_base = 0;
  pl->merge_rows_all = 0;
  pl->merge_rows_multi = 0;
  pl->num_multi = 0;
  pl->max_rows = 0;
  for (int32_t s = 0; s < S; ++s) {
    SeqRec& r = pl->seqs[s];
    r.kv_base = kv_base;
    r.q_base = q_base;
    r.n = pl->kv_lens[s];
    r.row_base = row_base;
    r.q = pl->q_lens[s];
    r.nb = int32_t((r.n + B - 1) / B);
    r.rows = r.q * g;
    r.pad = 0;
    kv_base += r.n;
    q_base += r.q;
    row_base += int64_t(r.nb) * Hkv * r.rows;
    pl->merge_rows_all += int64_t(Hkv) * r.rows;
    if (r.nb > 1) {
      pl->merge_rows_multi += int64_t(Hkv) * r.rows;
      pl->num_multi++;
    }
    pl->max_rows = std::max(pl->max_rows, r.rows);
  }
  pl->total_kv = kv_base;
  pl->total_q = q_base;
  pl->partial_rows = row_base;
  pl->ws_lse_offset = align16(uint64_t(row_base) * pl->D * sizeof(float));
  // The LSE area also holds the backward pass's two per-row values (D and the LSE in
  // base 2), 2 * sum_s q_s * Hq floats, more than the partial rows of one-block sequences.
  // The output area keeps its fp32 size with fp16 partials too: the backward pass puts
  // fp32 dQ parts there. With fp16 partials the LSE area holds (LSE, scale) pairs.
  const uint64_t lse_words = uint64_t(row_base) * (pl->pfmt == SPLITKV_PARTIAL_F16_ROWSCALE ? 2 : 1);
  pl->ws_bytes = pl->ws_lse_offset +
                 align16(std::max<uint64_t>(lse_words, 2 * uint64_t(q_base) * uint64_t(pl->Hq)) * sizeof(float));

  // Units in enumeration order, with their costs.
  pl->u_seq.clear();
  pl->u_block.clear();
  pl->u_kv.clear();
  pl->u_len.clear();
  pl->u_cost.clear();
  for (int32_t s = 0; s < S; ++s) {
    const SeqRec& r = pl->seqs[s];
    for (int32_t b = 0; b < r.nb; ++b) {
      const int32_t len = int32_t(std::min<int64_t>(B, r.n - int64_t(b) * B));
      // heads = g per KV-head unit or Hq = g * Hkv per whole-block unit.
      const int64_t rows = int64_t(r.q) * g;
      const int64_t cost = pl->ridge == 0 ? int64_t(r.q) * len * heads
                                          : int64_t(len) * std::max<int64_t>(rows, pl->ridge) * (heads / g);
      if (per_head) {
        for (int32_t k = 0; k < Hkv; ++k) {
          pl->u_seq.push_back(s);
          pl->u_block.push_back(b);
          pl->u_kv.push_back(k);
          pl->u_len.push_back(len);
          pl->u_cost.push_back(cost);
        }
      } else {
        pl->u_seq.push_back(s);
        pl->u_block.push_back(b);
        pl->u_kv.push_back(-1);
        pl->u_len.push_back(len);
        pl->u_cost.push_back(cost);
      }
    }
  }
  const int64_t n = int64_t(pl->u_cost.size());

  // LPT: stable sort by cost descending, then least-loaded worker (lowest index on ties).
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  const std::vector<int64_t>& cost = pl->u_cost;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });

  using Entry = std::pair<int64_t, int32_t>;  // (load, worker): lexicographic min = least load, lowest index
  std::vector<Entry> heap_storage;
  heap_storage.reserve(m);
  for (int32_t w = 0; w < m; ++w) heap_storage.emplace_back(0, w);
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap(std::greater<Entry>(),
                                                                           std::move(heap_storage));
  pl->worker_of.assign(n, -1);
  pl->load.assign(m, 0);
  std::vector<std::vector<int32_t>> lists(m);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t u = order[i];
    Entry e = heap.top();
    heap.pop();
    const int32_t w = e.second;
    pl->worker_of[u] = w;
    lists[w].push_back(u);
    pl->load[w] = e.first + cost[u];
    heap.emplace(pl->load[w], w);
  }
  pl->worker_ptr.assign(m + 1, 0);
  pl->worker_units.clear();
  pl->worker_units.reserve(n);
  for (int32_t w = 0; w < m; ++w) {
    pl->worker_units.insert(pl->worker_units.end(), lists[w].begin(), lists[w].end());
    pl->worker_ptr[w + 1] = int32_t(pl->worker_units.size());
  }

  // Statistics.
  pl->total_cost = 0;
  int64_t max_cost = 0;
  for (int64_t c : cost) {
    pl->total_cost += c;
    max_cost = std::max(max_cost, c);
  }
  pl->makespan = 0;
  for (int64_t l : pl->load) pl->makespan = std::max(pl->makespan, l);
  pl->lower_bound = std::max<int64_t>((pl->total_cost + m - 1) / m, max_cost);
  pl->imbalance = pl->total_cost == 0
                      ? 0.0
                      : double(int64_t(m) * pl->makespan - pl->total_cost) / double(pl->total_cost);

  // Placement of the plan's workers on the launch's workgroups: workgroup (slot) s runs
  // on XCD s % 8 (workgroups are dealt to the XCDs round-robin). Without XCD speeds,
  // slot s runs worker s. With them, the most loaded workers go to the slots of the
  // fastest XCDs: workers by load descending and slots by their XCD's speed descending
  // (ties by index), paired in order. The plan itself (which units each worker has)
  // does not change.
  pl->slot_worker.resize(m);
  std::iota(pl->slot_worker.begin(), pl->slot_worker.end(), 0);
  if (!pl->xcd_speed.empty()) {
    std::vector<int32_t> ws(m), ss(m);
    std::iota(ws.begin(), ws.end(), 0);
    std::iota(ss.begin(), ss.end(), 0);
    std::stable_sort(ws.begin(), ws.end(), [&](int32_t a, int32_t b) { return pl->load[a] > pl->load[b]; });
    std::stable_sort(ss.begin(), ss.end(),
                     [&](int32_t a, int32_t b) { return pl->xcd_speed[a % 8] > pl->xcd_speed[b % 8]; });
    for (int32_t i = 0; i < m; ++i) pl->slot_worker[ss[i]] = ws[i];
  }

  // Device image.
  ImageLayout& L = pl->layout;
  uint64_t off = 0;
  L.seqs = off;
  off = align16(off + sizeof(SeqRec) * uint64_t(S));
  L.units = off;
  off = align16(off + sizeof(UnitRec) * uint64_t(n));
  L.worker_ptr = off;
  off = align16(off + sizeof(int32_t) * uint64_t(m + 1));
  L.merge_all = off;
  off = align16(off + sizeof(int64_t) * uint64_t(S + 1));
  L.merge_multi = off;
  off = align16(off + sizeof(int32_t) * uint64_t(std::max(pl->num_multi, 1)));
  L.merge_multi_base = off;
  off = align16(off + sizeof(int64_t) * uint64_t(pl->num_multi + 1));
  const int64_t groups_all = (pl->merge_rows_all + kMergeRowsPerGroup - 1) / kMergeRowsPerGroup;
  const int64_t groups_multi = (pl->merge_rows_multi + kMergeRowsPerGroup - 1) / kMergeRowsPerGroup;
  L.merge_groups_all = off;
  off = align16(off + sizeof(MergeGroup) * uint64_t(std::max<int64_t>(groups_all, 1)));
  L.merge_groups_multi = off;
  off = align16(off + sizeof(MergeGroup) * uint64_t(std::max<int64_t>(groups_multi, 1)));
  pl->num_key_tiles = 0;
  for (int32_t s = 0; s < S; ++s)
    if (pl->seqs[s].rows > kFusedRows) pl->num_key_tiles += (pl->seqs[s].n + kDkvTileKeys - 1) / kDkvTileKeys;
  L.key_tiles = off;
  off = align16(off + sizeof(KeyTile) * uint64_t(std::max<int64_t>(pl->num_key_tiles, 1)));

  // Jobs of the bf16 kernel in LPT order (units by cost descending, ties in
  // enumeration order); a unit expands to its KV heads, each head to its row passes.
  // Each worker's static list holds the jobs of its units in its list order.
  std::vector<JobRec> jobs;
  std::vector<int32_t> unit_job(n + 1, 0);  // unit u's jobs start at unit_job[u]
  std::vector<int32_t> unit_njob(n, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t u = order[i];
    unit_job[u] = int32_t(jobs.size());
    const SeqRec& r = pl->seqs[pl->u_seq[u]];
    const int32_t b = pl->u_block[u];
    const int64_t key0 = int64_t(b) * B;
    const int32_t len = pl->u_len[u];
    // Query token i sees keys up to n - q + i, i.e. block keys t <= (n - q - key0) + i.
    const int32_t lim0 = pl->causal ? int32_t(std::min<int64_t>(len, r.n - r.q - key0)) : len;
    const int32_t nrt = (r.rows + 15) / 16;
    const int32_t kv_lo = per_head ? pl->u_kv[u] : 0, kv_hi = per_head ? kv_lo + 1 : Hkv;
    // Row passes of at most kPassTiles tiles, as even as possible (a unit's passes are
    // then alike, and run in the same launch).
    const int32_t npass = (nrt + kPassTiles - 1) / kPassTiles;
    for (int32_t kv = kv_lo; kv < kv_hi; ++kv) {
      for (int32_t pi = 0, t0 = 0; pi < npass; ++pi) {
        const int32_t tn = nrt / npass + (pi < nrt % npass ? 1 : 0);
        JobRec j{};
        j.kv_tok = r.kv_base + key0;
        j.q_tok = r.q_base;
        j.ws_row = r.row_base + (int64_t(kv) * r.nb + b) * r.rows;
        j.kv = kv;
        j.len = len;
        j.lim0 = lim0;
        j.rows = r.rows;
        j.tile_lo = t0;
        j.tile_n = tn;
        t0 += tn;
        const int32_t rmax = std::min(r.rows, t0 * 16) - 1;  // the pass's last row
        const int64_t tmax = std::min<int64_t>(len - 1, int64_t(lim0) + rmax / g);
        j.nst = tmax < 0 ? 1 : int32_t(tmax / kStageKeys) + 1;
        const int32_t wr_log = j.tile_n >= 8 ? 3 : j.tile_n >= 4 ? 2 : j.tile_n >= 2 ? 1 : 0;
        j.flags = wr_log | (r.rows <= kQTileRows ? kJobQTile : 0) | (r.nb == 1 ? kJobSingle : 0) |
                  (r.rows <= kFusedRows ? kJobFusedKV : 0);
        jobs.push_back(j);
      }
    }
    unit_njob[u] = int32_t(jobs.size()) - unit_job[u];
  }
  // Estimated job time, len * max(rows, 128): a job with few rows is bound by streaming
  // its block, one with many by the matrix cores.
  const int64_t nj = int64_t(jobs.size());
  std::vector<int64_t> jc(nj);
  for (int64_t i = 0; i < nj; ++i) {
    const JobRec& j = jobs[i];
    const int64_t rows = std::min<int64_t>(j.rows, int64_t(j.tile_lo + j.tile_n) * 16) - int64_t(j.tile_lo) * 16;
    jc[i] = std::max<int64_t>(rows, 128) * j.len;
  }
  // Jobs whose pass covers at least kMmaMinTiles row tiles run in their own launch
  // (partial_mma.hip); the rest in the launch of partial_bf16.hip. The two launches run
  // one after the other, so each workgroup's list has a part for each, balanced on its
  // own.
  std::vector<char> big(nj, 0);
  int32_t nbig = 0;
  for (int64_t i = 0; i < nj; ++i) {
    big[i] = jobs[i].tile_n >= kMmaMinTiles;
    nbig += big[i];
  }
  auto unit_big = [&](int64_t u) {
    int32_t c = 0;
    for (int32_t k = 0; k < unit_njob[u]; ++k) c += big[unit_job[u] + k];
    return c;
  };
  // Execution order of the lists of the other launch. Workgroups are spread over the
  // GPU's 8 XCDs round-robin (workgroup w on XCD w % 8), and the XCDs have their own L2.
  // A unit with several jobs (row passes, or KV heads of a whole-block unit) reads its
  // block once per job, so within each XCD class (workers w = x mod 8) the jobs of the
  // multi-job units assigned to its workers are shared by the class: taken in LPT
  // order, each goes to the class worker with the least estimated time so far (its own
  // single-job units counted first), and runs ahead of that worker's single-job units. A
  // unit's jobs then run at the same time on neighbouring workgroups of one XCD, and the
  // block is read from HBM about once; the class's workers stay balanced in estimated
  // time.
  std::vector<std::vector<int32_t>> lists_w(m), lists_big(m);
  const int32_t ncls = (m % 8 == 0 && m >= 16) ? 8 : 1;
  // A block read by one job, or by jobs dealt to distinct workers of one class (which
  // read it at about the same time), is not read again afterwards: its K/V loads carry
  // the non-temporal hint, so the streamed lines do not displace reused ones in L2.
  for (int64_t u = 0; u < n; ++u)
    if (unit_njob[u] == 1 || (ncls > 1 && unit_njob[u] <= m / ncls))
      for (int32_t k = 0; k < unit_njob[u]; ++k) jobs[unit_job[u] + k].flags |= kJobStream;
  typedef std::pair<int64_t, int32_t> LoadW;  // (estimated time, slot or class)
  for (int32_t x = 0; x < ncls; ++x) {
    std::vector<int32_t> shared;
    std::priority_queue<LoadW, std::vector<LoadW>, std::greater<LoadW>> heap;
    for (int32_t sl = x; sl < m; sl += ncls) {
      const int32_t w = pl->slot_worker[sl];
      int64_t own = 0;
      for (int32_t i = pl->worker_ptr[w]; i < pl->worker_ptr[w + 1]; ++i) {
        const int32_t u = pl->worker_units[i];
        const bool multi = unit_njob[u] - unit_big(u) > 1 && ncls > 1;
        for (int32_t k = 0; k < unit_njob[u]; ++k) {
          if (big[unit_job[u] + k]) continue;
          if (multi)
            shared.push_back(unit_job[u] + k);
          else
            own += jc[unit_job[u] + k];
        }
      }
      heap.push(LoadW(own, sl));
    }
    std::sort(shared.begin(), shared.end());  // job numbers follow the LPT order
    for (int32_t jn : shared) {
      LoadW e = heap.top();
      heap.pop();
      lists_w[e.second].push_back(jn);
      e.first += jc[jn];
      heap.push(e);
    }
    for (int32_t sl = x; sl < m; sl += ncls) {
      const int32_t w = pl->slot_worker[sl];
      for (int32_t i = pl->worker_ptr[w]; i < pl->worker_ptr[w + 1]; ++i) {
        const int32_t u = pl->worker_units[i];
        if (unit_njob[u] - unit_big(u) == 1 || ncls == 1)
          for (int32_t k = 0; k < unit_njob[u]; ++k)
            if (!big[unit_job[u] + k]) lists_w[sl].push_back(unit_job[u] + k);
      }
    }
  }
  // The matrix-path launch: the units' jobs in LPT order (unit cost descending), each
  // unit's jobs to the XCD class with the least estimated time so far (its passes then
  // share one L2), and within the class each job to the workgroup with the least
  // estimated time so far (ties to the lowest index).
  {
    std::vector<std::vector<int32_t>> cls_jobs(ncls);
    std::priority_queue<LoadW, std::vector<LoadW>, std::greater<LoadW>> ch;
    for (int32_t x = 0; x < ncls; ++x) ch.push(LoadW(0, x));
    for (int64_t i = 0; i < n; ++i) {
      const int32_t u = order[i];
      if (unit_big(u) == 0) continue;
      LoadW e = ch.top();
      ch.pop();
      for (int32_t k = 0; k < unit_njob[u]; ++k)
        if (big[unit_job[u] + k]) {
          cls_jobs[e.second].push_back(unit_job[u] + k);
          e.first += jc[unit_job[u] + k];
        }
      ch.push(e);
    }
    for (int32_t x = 0; x < ncls; ++x) {
      std::priority_queue<LoadW, std::vector<LoadW>, std::greater<LoadW>> heap;
      for (int32_t sl = x; sl < m; sl += ncls) heap.push(LoadW(0, sl));
      for (int32_t jn : cls_jobs[x]) {
        LoadW e = heap.top();
        heap.pop();
        lists_big[e.second].push_back(jn);
        e.first += jc[jn];
        heap.push(e);
      }
    }
  }
  // Job numbers: the matrix-path jobs first, then the others, each group in LPT order.
  std::vector<int32_t> perm(nj);
  {
    int32_t a = 0, b = nbig;
    for (int64_t i = 0; i < nj; ++i) perm[i] = big[i] ? a++ : b++;
    std::vector<JobRec> jobs2(nj);
    std::vector<int64_t> jc2(nj);
    for (int64_t i = 0; i < nj; ++i) {
      jobs2[perm[i]] = jobs[i];
      jc2[perm[i]] = jc[i];
    }
    jobs.swap(jobs2);
    jc.swap(jc2);
  }
  std::vector<int32_t> wjobs;
  wjobs.reserve(jobs.size());
  std::vector<int32_t> job_ptr(m + 1, 0), split_ptr(m, 0);
  for (int32_t w = 0; w < m; ++w) {
    for (int32_t jn : lists_big[w]) wjobs.push_back(perm[jn]);
    split_ptr[w] = int32_t(wjobs.size());
    for (int32_t jn : lists_w[w]) wjobs.push_back(perm[jn]);
    job_ptr[w + 1] = int32_t(wjobs.size());
  }
  for (int32_t w = 0; w < m; ++w) {
    lists_big[w].assign(wjobs.begin() + job_ptr[w], wjobs.begin() + split_ptr[w]);
    lists_w[w].assign(wjobs.begin() + split_ptr[w], wjobs.begin() + job_ptr[w + 1]);
  }
  pl->num_mma_jobs = nbig;
  pl->mma_partial_passes = false;
  for (int32_t i = 0; i < nbig; ++i)
    if (jobs[i].tile_n < kPassTiles) pl->mma_partial_passes = true;
  pl->num_jobs = int64_t(jobs.size());
  pl->num_fused_jobs = 0;
  for (const JobRec& j : jobs) pl->num_fused_jobs += (j.flags & kJobFusedKV) ? 1 : 0;
  // Queue schedule. The jobs at the end of the LPT order that make up the last fifth
  // of the estimated time form the shared tail, cut into chunks of consecutive jobs of
  // at least min(half the largest job, 1/32 of a worker's average) estimated time.
  // Chunk c is entry c / kQueues of sub-queue c % kQueues; workgroup w starts on
  // sub-queue w % kQueues (workgroups are spread over the XCDs round-robin, so each
  // sub-queue has one XCD's workgroups as first takers).
  {
    // Only jobs of the partial_bf16 launch (numbered from nbig on) take part.
    int64_t total = 0, maxc = 0;
    for (int64_t i = nbig; i < nj; ++i) {
      total += jc[i];
      maxc = std::max(maxc, jc[i]);
    }
    int64_t h = nj, acc = 0;
    while (h > nbig && acc * 5 < total) acc += jc[--h];
    pl->tail_start = int32_t(h);
    const int64_t target = std::max<int64_t>(1, std::min(maxc / 2, total / (int64_t(m) * 32)));
    pl->chunk_ptr.assign(1, int32_t(h));
    int64_t cur = 0;
    for (int64_t i = h; i < nj; ++i) {
      cur += jc[i];
      if (cur >= target) {
        pl->chunk_ptr.push_back(int32_t(i + 1));
        cur = 0;
      }
    }
    if (pl->chunk_ptr.back() != nj) pl->chunk_ptr.push_back(int32_t(nj));
    // Worth its synchronisation only with many jobs per workgroup.
    pl->queue_default = nj - nbig >= int64_t(16) * m;
  }
  // Modelled balance of the schedules as they execute (the LPT plan's own imbalance is
  // the assignment of units to workers). A job's share of the page's cost is its pass
  // rows * len (a unit's jobs add up to its q_s * len * heads). The two launches run one
  // after the other, so the modelled time is the sum of their largest workgroup loads:
  // imbalance = (m * (max_w big_w + max_w other_w) - total) / total.
  {
    auto imb = [&](const std::vector<int64_t>& a, const std::vector<int64_t>& b) {
      int64_t tot = 0, ma = 0, mb = 0;
      for (int32_t w = 0; w < m; ++w) {
        tot += a[w] + b[w];
        ma = std::max(ma, a[w]);
        mb = std::max(mb, b[w]);
      }
      return tot == 0 ? 0.0 : double(int64_t(m) * (ma + mb) - tot) / double(tot);
    };
    std::vector<int64_t> pc(nj);
    for (int64_t i = 0; i < nj; ++i) {
      const JobRec& j = jobs[i];
      const int64_t rows = std::min<int64_t>(j.rows, int64_t(j.tile_lo + j.tile_n) * 16) - int64_t(j.tile_lo) * 16;
      pc[i] = rows * j.len;
    }
    std::vector<int64_t> bc(m, 0), be(m, 0), lc(m, 0), le(m, 0);
    for (int32_t w = 0; w < m; ++w) {
      for (int32_t jn : lists_big[w]) {
        bc[w] += pc[jn];
        be[w] += jc[jn];
      }
      for (int32_t jn : lists_w[w]) {
        lc[w] += pc[jn];
        le[w] += jc[jn];
      }
    }
    pl->exec_static = imb(bc, lc);
    pl->exec_static_est = imb(be, le);
    // QUEUE: each workgroup's list without the shared tail, then the tail's chunks in
    // order, each to the workgroup with the least estimated time so far (lowest index on
    // ties): the run-time rule "next chunk to the first free workgroup" with the
    // planner's estimate as the time.
    std::priority_queue<std::pair<int64_t, int32_t>, std::vector<std::pair<int64_t, int32_t>>,
                        std::greater<std::pair<int64_t, int32_t>>>
        fr;
    std::vector<int64_t> lq(m, 0);
    for (int32_t w = 0; w < m; ++w) {
      for (int32_t jn : lists_w[w])
        if (jn < pl->tail_start) lq[w] += jc[jn];
      fr.emplace(lq[w], w);
    }
    for (size_t c = 0; c + 1 < pl->chunk_ptr.size(); ++c) {
      int64_t t = 0;
      for (int32_t jn = pl->chunk_ptr[c]; jn < pl->chunk_ptr[c + 1]; ++jn) t += jc[jn];
      auto e = fr.top();
      fr.pop();
      lq[e.second] = e.first + t;
      fr.emplace(lq[e.second], e.second);
    }
    pl->exec_queue_est = imb(be, lq);
  }
  L.jobs = off;
  off = align16(off + sizeof(JobRec) * jobs.size());
  L.wjobs = off;
  off = align16(off + sizeof(int32_t) * std::max<size_t>(wjobs.size(), 1));
  L.job_ptr = off;
  off = align16(off + sizeof(int32_t) * uint64_t(m + 1));
  L.split_ptr = off;
  off = align16(off + sizeof(int32_t) * uint64_t(m));
  L.chunk_ptr = off;
  off = align16(off + sizeof(int32_t) * pl->chunk_ptr.size());
  off = (off + 255) & ~uint64_t(255);
  L.sched = off;
  off += kSchedBytes;
  L.total = off;

  pl->image.assign(L.total, 0);
  uint8_t* base = pl->image.data();
  std::memcpy(base + L.seqs, pl->seqs.data(), sizeof(SeqRec) * S);
  // Units grouped by slot (the workers placed on the slots, in slot order).
  UnitRec* ur = reinterpret_cast<UnitRec*>(base + L.units);
  int32_t* sp = reinterpret_cast<int32_t*>(base + L.worker_ptr);
  sp[0] = 0;
  int64_t ui = 0;
  for (int32_t sl = 0; sl < m; ++sl) {
    const int32_t w = pl->slot_worker[sl];
    for (int32_t i = pl->worker_ptr[w]; i < pl->worker_ptr[w + 1]; ++i, ++ui) {
      const int32_t u = pl->worker_units[i];
      ur[ui].seq = pl->u_seq[u];
      ur[ui].block = pl->u_block[u];
      ur[ui].kv0 = per_head ? pl->u_kv[u] : 0;
      ur[ui].nkv = per_head ? 1 : Hkv;
    }
    sp[sl + 1] = int32_t(ui);
  }
  int64_t* ma = reinterpret_cast<int64_t*>(base + L.merge_all);
  int32_t* mm = reinterpret_cast<int32_t*>(base + L.merge_multi);
  int64_t* mb = reinterpret_cast<int64_t*>(base + L.merge_multi_base);
  ma[0] = 0;
  mb[0] = 0;
  int32_t j = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t rows = int64_t(Hkv) * pl->seqs[s].rows;
    ma[s + 1] = ma[s] + rows;
    if (pl->seqs[s].nb > 1) {
      mm[j] = s;
      mb[j + 1] = mb[j] + rows;
      ++j;
    }
  }
  // Merge workgroups' sequences (every sequence has at least one row, so the prefixes
  // rise strictly and a row's sequence is unique).
  auto fill_groups = [&](MergeGroup* out, const int64_t* prefix, const int32_t* ids, int32_t count, int64_t total) {
    int32_t lo = 0;
    for (int64_t g0 = 0; g0 < total; g0 += kMergeRowsPerGroup) {
      while (prefix[lo + 1] <= g0) ++lo;
      const int64_t last = std::min<int64_t>(g0 + kMergeRowsPerGroup, total) - 1;
      MergeGroup& e = out[g0 / kMergeRowsPerGroup];
      e.lo_cross = lo | (last >= prefix[lo + 1] ? kMergeCross : 0);
      e.seq = ids ? ids[lo] : lo;
    }
    (void)count;
  };
  fill_groups(reinterpret_cast<MergeGroup*>(base + L.merge_groups_all), ma, nullptr, S, pl->merge_rows_all);
  KeyTile* kt = reinterpret_cast<KeyTile*>(base + L.key_tiles);
  for (int32_t s = 0; s < S; ++s) {
    if (pl->seqs[s].rows <= kFusedRows) continue;
    const int64_t nt = (pl->seqs[s].n + kDkvTileKeys - 1) / kDkvTileKeys;
    for (int64_t t = 0; t < nt; ++t, ++kt) {
      kt->seq = s;
      kt->tile = int32_t(t);
    }
  }
  fill_groups(reinterpret_cast<MergeGroup*>(base + L.merge_groups_multi), mb, mm, pl->num_multi, pl->merge_rows_multi);
  if (!jobs.empty()) std::memcpy(base + L.jobs, jobs.data(), sizeof(JobRec) * jobs.size());
  if (!wjobs.empty()) std::memcpy(base + L.wjobs, wjobs.data(), sizeof(int32_t) * wjobs.size());
  std::memcpy(base + L.job_ptr, job_ptr.data(), sizeof(int32_t) * (m + 1));
  std::memcpy(base + L.split_ptr, split_ptr.data(), sizeof(int32_t) * m);
  std::memcpy(base + L.chunk_ptr, pl->chunk_ptr.data(), sizeof(int32_t) * pl->chunk_ptr.size());
  // The scheduling area (L.sched) stays zero: launches leave it that way.
}

}  // namespace splitkv
