// Host-side task-graph builder: tiles one decode step into per-CU instruction
// streams and proves the schedule covers every weight exactly once and cannot
// deadlock.  The per-CU streams with dependency counters in place of
// grid-wide barriers follow the ForgeMegakernel milestones ("4.1 The universal
// knowledge base and the milestones": per-SM instruction streams, dependency
// counters, buffer pool); the one-block-per-SM task-descriptor execution model
// follows the Cohere megakernel digest.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

namespace {

int stage_rows(const PlanCfg& p, int st) {
  switch (st) {
    case ST_QKV: return (p.nq + 2 * p.nkv) * p.hd;
    case ST_O: return p.d;
    case ST_GU: return 2 * p.I;
    case ST_DOWN: return p.d;
    case ST_LM: return p.V;
  }
  return 0;
}

int stage_k(const PlanCfg& p, int st) {
  switch (st) {
    case ST_QKV: return p.d;
    case ST_O: return p.nq * p.hd;
    case ST_GU: return p.d;
    case ST_DOWN: return p.I;
    case ST_LM: return p.d;
  }
  return 0;
}

// K-slice boundary i of nks, aligned to 64 elements.
int kbound(int K, int nks, int i) {
  if (i >= nks) return K;
  long long u = (long long)(K / 64) * i / nks;
  return (int)(u * 64);
}

struct Choice {
  int R = 1, nks = 1;
  double cost = 1e300;
};

Choice choose_tiling(const PlanCfg& p, int M, int K, int batch, bool mfma) {
  Choice best;
  const int Rs_mfma[3] = {4, 2, 1};
  const int Rs_valu[1] = {1};
  const int* Rs = mfma ? Rs_mfma : Rs_valu;
  int nR = mfma ? 3 : 1;
  for (int ri = 0; ri < nR; ++ri) {
    int R = Rs[ri];
    long long groups = (M + 16 * R - 1) / (16 * R);
    for (int nks = 1; nks <= 64; ++nks) {
      if (K / nks < 64) break;
      int kmax = 0;
      for (int i = 0; i < nks; ++i) kmax = std::max(kmax, kbound(K, nks, i + 1) - kbound(K, nks, i));
      if ((long long)batch * kmax * 2 > p.xb_bytes) continue;
      long long units = groups * nks;
      long long per_cu = (units + p.ncu - 1) / p.ncu;
      // bytes streamed by the busiest CU plus a per-task overhead expressed in
      // bytes (reduction, epilogue, signal); split-K adds a partial round trip.
      double unit_bytes = 16.0 * R * kmax * 2.0;
      double overhead = 12288.0 + (nks > 1 ? 16384.0 : 0.0);
      double cost = per_cu * (unit_bytes + overhead);
      if (cost < best.cost * 0.999) {
        best.cost = cost;
        best.R = R;
        best.nks = nks;
      }
    }
  }
  return best;
}

int owner(long long u, long long units, int ncu) { return (int)(u * ncu / units); }

}  // namespace

void free_plan(Plan* p) {
  if (!p) return;
  free(p->tasks);
  free(p->task_off);
  free(p->expect);
  p->tasks = nullptr;
  p->task_off = nullptr;
  p->expect = nullptr;
}

int build_plan(const PlanCfg& pc, int batch, Plan* out) {
  if (batch < 1 || batch > kMaxBatch || pc.ncu < 1) return MK_ERR_INVALID_ARG;
  const int ncu = pc.ncu;
  const bool mfma = batch >= pc.mfma_min_batch;
  std::vector<std::vector<Task>> S(ncu);
  Plan P;
  P.batch = batch;
  P.mfma = mfma ? 1 : 0;
  P.n_counters = n_counters(pc.L);
  std::vector<long long> cu_bytes(ncu, 0);
  int part_blocks = 0, grp_counters = 0;

  auto base_task = [](int type, int stage, int layer) {
    Task t;
    memset(&t, 0, sizeof(t));
    t.type = type;
    t.stage = stage;
    t.layer = layer;
    t.group = -1;
    t.part_slot = -1;
    t.wait_ctr = -1;
    t.signal_ctr = -1;
    t.nks = 1;
    return t;
  };

  // Embedding gather: 64 columns per task.
  {
    int n = pc.d / 64;
    for (int i = 0; i < n; ++i) {
      Task t = base_task(TT_EMBED, ST_EMBED, 0);
      t.row0 = 64 * i;
      t.nsub = 64;
      t.signal_ctr = ctr_embed();
      S[owner(i, n, ncu)].push_back(t);
    }
  }

  // GEMV stages: choose a tiling per stage kind once (the same for all layers).
  Choice ch[6];
  int grp_base[6] = {0, 0, 0, 0, 0, 0};
  int part_base[6] = {0, 0, 0, 0, 0, 0};
  const int gemv_stages[5] = {ST_QKV, ST_O, ST_GU, ST_DOWN, ST_LM};
  for (int si = 0; si < 5; ++si) {
    int st = gemv_stages[si];
    ch[st] = choose_tiling(pc, stage_rows(pc, st), stage_k(pc, st), batch, mfma);
    int groups = (stage_rows(pc, st) + 16 * ch[st].R - 1) / (16 * ch[st].R);
    if (ch[st].nks > 1) {
      grp_base[st] = grp_counters;
      grp_counters += groups;
      part_base[st] = part_blocks;
      part_blocks += groups * ch[st].nks;
    }
    P.stage_ksplit[st] = ch[st].nks;
    P.stage_rows[st] = 16 * ch[st].R;
  }
  P.stage_ksplit[ST_ATTN] = 0;
  P.stage_rows[ST_ATTN] = 0;

  auto emit_gemv = [&](int st, int layer, int wait, int signal) {
    const int M = stage_rows(pc, st), K = stage_k(pc, st);
    const Choice& c = ch[st];
    const long long groups = (M + 16 * c.R - 1) / (16 * c.R);
    const long long units = groups * c.nks;
    for (long long u = 0; u < units; ++u) {
      int g = (int)(u / c.nks), ks = (int)(u % c.nks);
      Task t = base_task(TT_GEMV, st, layer);
      t.row0 = g * 16 * c.R;
      t.nsub = c.R;
      t.k0 = kbound(K, c.nks, ks);
      t.k1 = kbound(K, c.nks, ks + 1);
      t.ks = ks;
      t.nks = c.nks;
      t.group = c.nks > 1 ? g : -1;
      t.part_slot = c.nks > 1 ? part_base[st] + g * c.nks : -1;
      t.wait_ctr = wait;
      t.signal_ctr = signal;
      int ks_len = t.k1 - t.k0;
      if (mfma) {
        int steps = ks_len / 32;
        t.nchunks = (steps * c.R + kWaveLoads - 1) / kWaveLoads;
      } else {
        t.nchunks = (ks_len + kValuBlock - 1) / kValuBlock;
      }
      int rows = std::min(16 * c.R, M - t.row0);
      int cu = owner(u, units, ncu);
      cu_bytes[cu] += (long long)rows * ks_len * 2;
      S[cu].push_back(t);
    }
  };

  for (int l = 0; l < pc.L; ++l) {
    int wait_in = l == 0 ? ctr_embed() : ctr_stage(l - 1, ST_DOWN);
    emit_gemv(ST_QKV, l, wait_in, ctr_stage(l, ST_QKV));
    for (int c = 0; c < ncu; ++c) {
      Task t = base_task(TT_ATTN, ST_ATTN, l);
      t.wait_ctr = ctr_stage(l, ST_QKV);
      t.signal_ctr = ctr_stage(l, ST_ATTN);
      S[c].push_back(t);
    }
    emit_gemv(ST_O, l, ctr_stage(l, ST_ATTN), ctr_stage(l, ST_O));
    emit_gemv(ST_GU, l, ctr_stage(l, ST_O), ctr_stage(l, ST_GU));
    emit_gemv(ST_DOWN, l, ctr_stage(l, ST_GU), ctr_stage(l, ST_DOWN));
  }
  emit_gemv(ST_LM, pc.L, ctr_stage(pc.L - 1, ST_DOWN), ctr_lm(pc.L));

  // Flatten, count expected signals per counter shard.
  std::vector<int> expect((size_t)P.n_counters * kShards, 0);
  std::vector<int> total_signals(P.n_counters, 0);
  int n_tasks = 0, max_tasks = 0;
  for (int c = 0; c < ncu; ++c) {
    n_tasks += (int)S[c].size();
    max_tasks = std::max(max_tasks, (int)S[c].size());
    for (const Task& t : S[c]) {
      if (t.signal_ctr >= 0) {
        expect[(size_t)t.signal_ctr * kShards + (c % kShards)] += 1;
        total_signals[t.signal_ctr] += 1;
      }
    }
  }

  // ---- validation --------------------------------------------------------
  // (1) every (group, k-slice) unit of every GEMV stage exactly once, and
  //     every staged input slice fits the LDS staging buffer.
  for (int l = 0; l <= pc.L; ++l) {
    for (int si = 0; si < 5; ++si) {
      int st = gemv_stages[si];
      if ((st == ST_LM) != (l == pc.L)) continue;
      const Choice& c = ch[st];
      long long groups = (stage_rows(pc, st) + 16 * c.R - 1) / (16 * c.R);
      std::vector<int> seen(groups * c.nks, 0);
      long long covered = 0;
      for (int cu = 0; cu < ncu; ++cu)
        for (const Task& t : S[cu]) {
          if (t.type != TT_GEMV || t.stage != st || t.layer != l) continue;
          long long g = t.row0 / (16 * c.R);
          seen[g * c.nks + t.ks] += 1;
          covered += (long long)std::min(16 * c.R, stage_rows(pc, st) - t.row0) * (t.k1 - t.k0);
          if ((long long)batch * (t.k1 - t.k0) * 2 > pc.xb_bytes) return MK_ERR_PLAN;
        }
      for (int v : seen)
        if (v != 1) return MK_ERR_PLAN;
      if (covered != (long long)stage_rows(pc, st) * stage_k(pc, st)) return MK_ERR_PLAN;
    }
  }
  // (2) deadlock freedom: execute the in-order streams abstractly; a task may
  //     run once every signal of the counter it waits on has been given.
  {
    std::vector<int> given(P.n_counters, 0);
    std::vector<size_t> pc_(ncu, 0);
    size_t done = 0;
    bool progress = true;
    while (progress) {
      progress = false;
      for (int c = 0; c < ncu; ++c) {
        while (pc_[c] < S[c].size()) {
          const Task& t = S[c][pc_[c]];
          if (t.wait_ctr >= 0 && given[t.wait_ctr] < total_signals[t.wait_ctr]) break;
          if (t.signal_ctr >= 0) given[t.signal_ctr] += 1;
          pc_[c] += 1;
          done += 1;
          progress = true;
        }
      }
    }
    if (done != (size_t)n_tasks) return MK_ERR_PLAN;
  }

  // ---- stats & output ----------------------------------------------------
  for (int si = 0; si < 5; ++si) {
    int st = gemv_stages[si];
    int layer = st == ST_LM ? pc.L : 0;
    std::vector<long long> b(ncu, 0);
    int nt = 0;
    for (int c = 0; c < ncu; ++c)
      for (const Task& t : S[c])
        if (t.type == TT_GEMV && t.stage == st && t.layer == layer) {
          b[c] += (long long)std::min(16 * t.nsub, stage_rows(pc, st) - t.row0) * (t.k1 - t.k0) * 2;
          nt++;
        }
    long long mx = 0, sum = 0;
    for (long long v : b) {
      mx = std::max(mx, v);
      sum += v;
    }
    double bal = mx > 0 ? (double)sum / ncu / mx : 1.0;
    P.balance_min = std::min(P.balance_min, bal);
    P.stage_tasks[st] = nt;
  }
  P.stage_tasks[ST_ATTN] = ncu;
  for (long long v : cu_bytes) {
    P.weight_bytes += v;
    P.max_cu_weight_bytes = std::max(P.max_cu_weight_bytes, v);
  }
  P.n_tasks = n_tasks;
  P.max_tasks_per_cu = max_tasks;
  P.part_blocks = part_blocks;
  P.grp_counters = grp_counters;
  for (int i = 0; i < 6; ++i) P.grp_off[i] = grp_base[i];
  P.tasks = (Task*)malloc(sizeof(Task) * (size_t)std::max(1, n_tasks));
  P.task_off = (int*)malloc(sizeof(int) * (size_t)(ncu + 1));
  P.expect = (int*)malloc(sizeof(int) * expect.size());
  if (!P.tasks || !P.task_off || !P.expect) {
    free_plan(&P);
    return MK_ERR_OOM;
  }
  int k = 0;
  for (int c = 0; c < ncu; ++c) {
    P.task_off[c] = k;
    for (const Task& t : S[c]) P.tasks[k++] = t;
  }
  P.task_off[ncu] = k;
  memcpy(P.expect, expect.data(), sizeof(int) * expect.size());
  *out = P;
  return MK_OK;
}

}  // namespace mk
