// Host-side task-graph builder: tiles one decode step into per-CU instruction
// streams and proves the schedule covers every weight exactly once and cannot
// deadlock.  The per-CU streams with fine-grained dependencies in place of
// grid-wide barriers follow the ForgeMegakernel milestones ("4.1 The universal
// knowledge base and the milestones": per-SM instruction streams, dependency
// counters, buffer pool); the one-block-per-SM task-descriptor execution model
// follows the Cohere megakernel digest.  On the device the hand-offs poll
// step-tagged data and only the LM head's completion is counted; the deadlock
// check here models every device wait as a wait on all of its possible
// producers (the schedule validator of the AutoMegaKernel page: deadlock
// freedom proven before anything runs).
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

// A GEMV stage is tiled into 16-row sub-tiles over 512-wide K blocks, in one
// of two ways:
//  * row-owner: each CU owns a contiguous range of whole sub-tiles over the
//    full K, cut into tasks of at most 4 x tiles_per_wave sub-tiles (wave w
//    owns sub-tiles w, w+4, ...).  Nothing is split, so a task's epilogue
//    runs straight from registers.
//  * stream-K: columns = (row group of `gs` sub-tiles) x (K block) are dealt
//    to CUs as equal contiguous ranges; a CU's range is cut into tasks at
//    row-group boundaries, and a row group whose K range is split over
//    several CUs is finished by the last of its pieces.
// The cheaper one is chosen per stage.  Costs are in units of one streamed
// 16 KB weight chunk on the busiest CU: a split is charged PlanCfg::split_chunks of
// extra latency; staging the activation slice a task reads (b x K range,
// 4 bytes per element in LDS) is charged per byte and per LDS window (each
// window is a barrier plus a memory round trip while the ring sits full;
// PlanCfg::window_chunks, 6 by default: on Llama-3.2-1B at batch 8 and
// Llama-3-8B at batch 1 a charge of 4 kept row-owner QKV / gate-up tilings
// that measured 5% and 3% slower per step than the stream-K ones 6 picks).
constexpr double kStageChunksPerChunk = 0.5;  // staged activation bytes, per 16 KB

struct Tiling {
  bool owner = false;
  bool ks = false;     // K-split: S K pieces of at most one LDS window each, dealt K-major
  int S = 1;           // K-split: pieces
  int gs = 4;          // stream-K: sub-tiles per group
  int tmax = 4;        // row-owner: sub-tiles per task
  int nst = 1;         // sub-tiles of the stage
  int nkb = 1;         // K blocks
  int ngroups = 1;     // stream-K groups
  long long ncols = 1;
};

Tiling tile_stage(const PlanCfg& p, int st, int M, int K, int tpw, int b) {
  const int mode = p.stage_mode[st] ? p.stage_mode[st] : p.gemv_mode;
  const int nst = (M + 15) / 16, nkb = (K + kKBlock - 1) / kKBlock;
  // K blocks of one LDS staging window at this batch (the kernel's rule)
  const int wkb = std::max(1, ((p.xb_bytes / (4 * b)) - 8) / kKBlock);
  // staging cost of one task over `kbs` K blocks
  auto stage_cost = [&](long long kbs) {
    const long long windows = (kbs + wkb - 1) / wkb;
    return (double)b * (double)kbs * kKBlock * 4.0 / kChunkBytes * kStageChunksPerChunk + (double)windows * p.window_chunks;
  };
  Tiling best;
  best.nst = nst;
  best.nkb = nkb;
  double best_cost = 1e300;
  for (int gs = kGroupSub; gs >= 1; gs >>= 1) {
    if (mode == 3 && gs != 1) continue;
    Tiling t = best;
    t.gs = gs;
    t.ngroups = (nst + gs - 1) / gs;
    t.ncols = (long long)t.ngroups * nkb;
    long long per_cu = (t.ncols + p.ncu - 1) / p.ncu;
    const bool split = (t.ncols % p.ncu) != 0 || ((t.ncols / p.ncu) % nkb) != 0;
    // a CU's columns touch at least one group: one staged slice per group touched
    const long long groups_cu = std::max(1LL, (per_cu + nkb - 1) / nkb);
    double cost = (double)per_cu * gs + 0.25 * (double)per_cu / nkb + (gs < kGroupSub ? 0.01 : 0.0) +
                  (split ? p.split_chunks : 0) + stage_cost(std::min<long long>(per_cu, nkb)) * (double)groups_cu;
    if (cost < best_cost) {
      best_cost = cost;
      best = t;
    }
  }
  Tiling own = best;
  own.owner = true;
  own.tmax = 4 * tpw;
  const long long tiles_cu = (nst + p.ncu - 1) / p.ncu;
  const long long tasks_cu = (tiles_cu + own.tmax - 1) / own.tmax;
  // a task whose full K fits one window reuses the slice staged by the CU's
  // previous task; otherwise every task stages all its windows again
  const double own_stage = stage_cost(nkb) * (double)(nkb <= wkb ? 1 : tasks_cu);
  const double own_cost = (double)tiles_cu * nkb + 0.25 * (double)tasks_cu + own_stage;
  const bool use_owner = mode == 1 || (mode == 0 && own_cost <= best_cost);
  // K-split: when a task's K range needs more than one staging window, cut K
  // into S pieces of at most one window each and deal (piece, sub-tile) units
  // K-major over the CUs, so each CU stages one input slice and streams its
  // units against it; every piece publishes its partial tile and a finish
  // task per CU sums the pieces of its share of the sub-tiles.  Restaging a
  // window costs a memory round trip per window and reads the whole input on
  // every CU; the pieces cost one 1 KB partial tile per (piece, sub-tile).
  // Worth it only when the tiling it replaces restages many windows per task
  // (measured: with 1-block windows at batch 16, 7-10 windows per task gained
  // 13% and the O projection's 4 gained 2%; at batch 8-9, 2-3 windows of 2-3
  // blocks each lost 4-8%).
  const Tiling& rep = use_owner ? own : best;
  const long long rep_kbs = rep.owner ? nkb : std::min<long long>(nkb, (rep.ncols + p.ncu - 1) / p.ncu);
  const long long rep_windows = (rep_kbs + wkb - 1) / wkb;
  if (p.ksplit && mode == 0 && nkb > wkb && rep_windows >= p.ksplit_min_windows) {
    Tiling k = own;
    k.owner = false;
    k.ks = true;
    k.S = (nkb + wkb - 1) / wkb;
    return k;
  }
  return use_owner ? own : best;
}

// first K block of piece s when nkb blocks are cut into S pieces
int piece_kb(int s, int nkb, int S) { return (int)((long long)s * nkb / S); }

int owner(long long u, long long units, int ncu) { return (int)(u * ncu / units); }

}  // namespace

void free_plan(Plan* p) {
  if (!p) return;
  free(p->tasks);
  free(p->task_off);
  free(p->expect);
  free(p->attn_map);
  p->attn_map = nullptr;
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
      t.flags = kTaskSignal;
      S[owner(i, n, ncu)].push_back(t);
    }
  }

  // GEMV stages: choose a tiling per stage kind once (the same for all layers).
  Tiling tl[6];
  int grp_base[6] = {0, 0, 0, 0, 0, 0};
  int part_base[6] = {0, 0, 0, 0, 0, 0};
  const int gemv_stages[5] = {ST_QKV, ST_O, ST_GU, ST_DOWN, ST_LM};
  // pieces of each group, identical for every layer of a stage
  std::vector<std::vector<int>> group_pieces(6);
  const int tpw = tiles_per_wave(mfma ? 0 : batch);
  for (int si = 0; si < 5; ++si) {
    int st = gemv_stages[si];
    tl[st] = tile_stage(pc, st, stage_rows(pc, st), stage_k(pc, st), tpw, batch);
    const Tiling& T = tl[st];
    P.stage_owner[st] = T.owner ? 1 : 0;
    if (T.ks) {
      // one 256-float tile slot per (sub-tile, piece), in 1024-float blocks
      group_pieces[st].assign(1, T.S);
      grp_base[st] = grp_counters;
      part_base[st] = part_blocks;
      part_blocks += (T.nst * T.S + 3) / 4;
      P.stage_ksplit[st] = T.S;
      P.stage_kpieces[st] = T.S;
      P.stage_rows[st] = 16 * T.tmax;
      continue;
    }
    if (T.owner) {
      group_pieces[st].assign(1, 1);
      grp_base[st] = grp_counters;
      part_base[st] = part_blocks;
      P.stage_ksplit[st] = 1;
      P.stage_rows[st] = 16 * T.tmax;
      continue;
    }
    group_pieces[st].assign(T.ngroups, 0);
    for (int c = 0; c < ncu; ++c) {
      long long c0 = T.ncols * c / ncu, c1 = T.ncols * (c + 1) / ncu;
      for (long long col = c0; col < c1;) {
        int g = (int)(col / T.nkb);
        long long gend = std::min(c1, (long long)(g + 1) * T.nkb);
        group_pieces[st][g] += 1;
        col = gend;
      }
    }
    int split_groups = 0, split_pieces = 0;
    for (int v : group_pieces[st])
      if (v > 1) {
        split_groups++;
        split_pieces += v;
      }
    grp_base[st] = grp_counters;
    grp_counters += T.ngroups;
    part_base[st] = part_blocks;
    part_blocks += split_pieces;
    int maxp = 1;
    for (int v : group_pieces[st]) maxp = std::max(maxp, v);
    P.stage_ksplit[st] = maxp;
    P.stage_rows[st] = 16 * T.gs;
    (void)split_groups;
  }
  P.stage_ksplit[ST_ATTN] = 0;
  P.stage_rows[ST_ATTN] = 0;
  // partial-block base of each split group (same layout for every layer)
  std::vector<std::vector<int>> group_part(6);
  for (int si = 0; si < 5; ++si) {
    int st = gemv_stages[si];
    if (tl[st].owner || tl[st].ks) continue;
    group_part[st].assign(tl[st].ngroups, -1);
    int nxt = part_base[st];
    for (int g = 0; g < tl[st].ngroups; ++g)
      if (group_pieces[st][g] > 1) {
        group_part[st][g] = nxt;
        nxt += group_pieces[st][g];
      }
  }

  // CUs that ran a task of the stage emitted last: a stage that left some CUs
  // idle finishes on the others, so the next row-owner stage avoids them
  // (its tasks then wait for their inputs on CUs that are already free)
  // unless that raises its tiles per CU by skip_prev or more.
  std::vector<char> prev_used(ncu, 1);
  std::vector<int> attn_map((size_t)pc.L * (ncu + 1), 0);
  auto emit_gemv = [&](int st, int layer, int wait, int signal) {
    const int M = stage_rows(pc, st), K = stage_k(pc, st);
    const Tiling& T = tl[st];
    const int nst = (M + 15) / 16;
    if (T.ks) {
      // units (piece s, sub-tile u), s-major.  With at least as many CUs as
      // pieces, piece s gets CUs [s ncu / S, (s+1) ncu / S) and its sub-tiles
      // are split evenly over them, so no CU stages two input windows (a CU
      // whose units straddled two pieces restaged and ran ~9 us behind the
      // others at Llama-2-13B b16, for at most one unit more per CU this
      // way); otherwise the units are dealt evenly over the CUs.  A CU's run
      // of units with one s becomes tasks of at most tmax sub-tiles.
      const long long units = (long long)T.S * nst;
      const bool aligned = ncu >= T.S && pc.ksplit_aligned;
      std::fill(prev_used.begin(), prev_used.end(), 1);
      for (int c = 0; c < ncu; ++c) {
        long long u0 = units * c / ncu, u1 = units * (c + 1) / ncu;
        if (aligned) {
          const int sp = (int)((long long)c * T.S / ncu);
          const int ca = (int)(((long long)sp * ncu + T.S - 1) / T.S), cb = (int)(((long long)(sp + 1) * ncu + T.S - 1) / T.S);
          u0 = (long long)sp * nst + (long long)nst * (c - ca) / (cb - ca);
          u1 = (long long)sp * nst + (long long)nst * (c + 1 - ca) / (cb - ca);
        }
        for (long long x = u0; x < u1;) {
          const int sp = (int)(x / nst), ua = (int)(x % nst);
          const int ub = (int)std::min<long long>(nst, ua + (u1 - x));
          for (int a = ua; a < ub; a += T.tmax) {
            const int e = std::min(ub, a + T.tmax);
            const int kb0 = piece_kb(sp, T.nkb, T.S), kb1 = piece_kb(sp + 1, T.nkb, T.S);
            Task t = base_task(TT_GEMV, st, layer);
            t.row0 = 16 * a;
            t.nsub = e - a;
            t.k0 = kb0 * kKBlock;
            t.k1 = std::min(K, kb1 * kKBlock);
            t.nks = T.S;
            t.ks = sp;
            t.part_slot = part_base[st] * 4;
            t.wait_ctr = wait;
            t.flags = kTaskPublish;
            t.nchunks = t.nsub * (kb1 - kb0);
            cu_bytes[c] += (long long)std::min(16 * t.nsub, M - t.row0) * (t.k1 - t.k0) * 2;
            S[c].push_back(t);
          }
          x += ub - ua;
        }
      }
      // finish tasks: CU c sums the pieces of sub-tiles [nst c / ncu, nst (c+1) / ncu)
      for (int c = 0; c < ncu; ++c) {
        const int f0 = (int)((long long)nst * c / ncu), f1 = (int)((long long)nst * (c + 1) / ncu);
        if (f1 <= f0) continue;
        Task t = base_task(TT_FIN, st, layer);
        t.row0 = 16 * f0;
        t.nsub = f1 - f0;
        t.k0 = 0;
        t.k1 = K;
        t.nks = T.S;
        t.part_slot = part_base[st] * 4;
        t.wait_ctr = wait;
        // only the LM head counts its completed tasks (for the greedy tokens)
        if (st == ST_LM) {
          t.signal_ctr = signal;
          t.flags = kTaskSignal;
        }
        S[c].push_back(t);
      }
      return;
    }
    if (T.owner) {
      std::vector<int> cus;
      int nprev = 0;
      for (int c = 0; c < ncu; ++c) nprev += prev_used[c];
      if (pc.skip_prev > 0 && nprev < ncu) {
        const int nfree = ncu - nprev;
        const int per_all = (nst + ncu - 1) / ncu, per_free = (nst + nfree - 1) / nfree;
        if (per_free - per_all < pc.skip_prev)
          for (int c = 0; c < ncu; ++c)
            if (!prev_used[c]) cus.push_back(c);
      }
      if (cus.empty())
        for (int c = 0; c < ncu; ++c) cus.push_back(c);
      const int nc = (int)cus.size();
      std::fill(prev_used.begin(), prev_used.end(), 0);
      for (int ci = 0; ci < nc; ++ci) {
        const int c = cus[ci];
        const int t0 = (int)((long long)nst * ci / nc), t1 = (int)((long long)nst * (ci + 1) / nc);
        if (t1 <= t0) continue;
        prev_used[c] = 1;
        const int n = t1 - t0, ntask = (n + T.tmax - 1) / T.tmax;
        for (int k = 0; k < ntask; ++k) {
          const int a = t0 + n * k / ntask, e = t0 + n * (k + 1) / ntask;
          Task t = base_task(TT_GEMV, st, layer);
          t.row0 = 16 * a;
          t.nsub = e - a;
          t.k0 = 0;
          t.k1 = K;
          t.wait_ctr = wait;
          t.signal_ctr = signal;
          t.nchunks = t.nsub * T.nkb;
          cu_bytes[c] += (long long)std::min(16 * t.nsub, M - t.row0) * K * 2;
          if (k == ntask - 1) t.flags |= kTaskSignal;
          S[c].push_back(t);
        }
      }
      return;
    }
    std::vector<int> seen(T.ngroups, 0);
    std::fill(prev_used.begin(), prev_used.end(), 1);
    for (int c = 0; c < ncu; ++c) {
      long long c0 = T.ncols * c / ncu, c1 = T.ncols * (c + 1) / ncu;
      int first = (int)S[c].size();
      for (long long col = c0; col < c1;) {
        int g = (int)(col / T.nkb);
        int kb_a = (int)(col - (long long)g * T.nkb);
        long long gend = std::min(c1, (long long)(g + 1) * T.nkb);
        int kb_b = (int)(gend - (long long)g * T.nkb);
        Task t = base_task(TT_GEMV, st, layer);
        t.row0 = g * 16 * T.gs;
        t.nsub = std::min(T.gs, nst - g * T.gs);
        t.k0 = kb_a * kKBlock;
        t.k1 = std::min(K, kb_b * kKBlock);
        t.nks = group_pieces[st][g];
        t.ks = seen[g]++;
        t.group = g;
        t.part_slot = t.nks > 1 ? group_part[st][g] : -1;
        t.wait_ctr = wait;
        t.signal_ctr = signal;
        t.nchunks = t.nsub * (kb_b - kb_a);
        int rows = std::min(16 * t.nsub, M - t.row0);
        cu_bytes[c] += (long long)rows * (t.k1 - t.k0) * 2;
        S[c].push_back(t);
        col = gend;
      }
      if ((int)S[c].size() > first) S[c].back().flags |= kTaskSignal;
    }
  };

  for (int l = 0; l < pc.L; ++l) {
    int wait_in = l == 0 ? ctr_embed() : ctr_stage(l - 1, ST_DOWN);
    emit_gemv(ST_QKV, l, wait_in, ctr_stage(l, ST_QKV));
    // attention slots: the CUs this layer's QKV stage left idle come first
    // (they wait for q/k/v with their cached rows already loaded); the
    // device caps the CUs at the idle ones when that keeps pieces short
    {
      int* m = &attn_map[(size_t)l * (ncu + 1)];
      int k = 0, nidle = 0;
      for (int c = 0; c < ncu; ++c)
        if (!prev_used[c]) m[c] = k++;
      nidle = k;
      for (int c = 0; c < ncu; ++c)
        if (prev_used[c]) m[c] = k++;
      m[ncu] = (pc.attn_idle && nidle >= ncu / 8 && nidle < ncu) ? nidle : 0;
      // the next stage treats the CUs attention runs on as the busy ones
      if (m[ncu] > 0)
        for (int c = 0; c < ncu; ++c) prev_used[c] = !prev_used[c];
      else
        std::fill(prev_used.begin(), prev_used.end(), 1);
    }
    for (int c = 0; c < ncu; ++c) {
      Task t = base_task(TT_ATTN, ST_ATTN, l);
      t.wait_ctr = ctr_stage(l, ST_QKV);
      t.signal_ctr = ctr_stage(l, ST_ATTN);
      t.flags = kTaskSignal;
      S[c].push_back(t);
    }
    emit_gemv(ST_O, l, ctr_stage(l, ST_ATTN), ctr_stage(l, ST_O));
    emit_gemv(ST_GU, l, ctr_stage(l, ST_O), ctr_stage(l, ST_GU));
    emit_gemv(ST_DOWN, l, ctr_stage(l, ST_GU), ctr_stage(l, ST_DOWN));
  }
  emit_gemv(ST_LM, pc.L, ctr_stage(pc.L - 1, ST_DOWN), ctr_lm(pc.L));

  // Flatten, count expected signals per counter shard.
  std::vector<int> expect((size_t)P.n_counters * kShards, 0);
  int n_tasks = 0, max_tasks = 0;
  for (int c = 0; c < ncu; ++c) {
    n_tasks += (int)S[c].size();
    max_tasks = std::max(max_tasks, (int)S[c].size());
    for (const Task& t : S[c]) {
      if (t.signal_ctr >= 0 && (t.flags & kTaskSignal)) {
        expect[(size_t)t.signal_ctr * kShards + (c % kShards)] += 1;
      }
    }
  }

  // ---- validation --------------------------------------------------------
  // (1) every (row, K element) of every GEMV stage is covered exactly once:
  //     per sub-tile, the K ranges of the tasks covering it tile [0, K) in
  //     piece order; split groups carry consistent piece indices; chunk
  //     counts match the task shapes; a K-split stage's sub-tiles are each
  //     finished by exactly one finish task.
  for (int l = 0; l <= pc.L; ++l) {
    for (int si = 0; si < 5; ++si) {
      int st = gemv_stages[si];
      if ((st == ST_LM) != (l == pc.L)) continue;
      const Tiling& T = tl[st];
      const int M = stage_rows(pc, st), K = stage_k(pc, st);
      const int nst = (M + 15) / 16;
      std::vector<int> next_k(nst, 0), pieces(nst, 0), fins(nst, 0);
      long long covered = 0;
      for (int cu = 0; cu < ncu; ++cu)
        for (const Task& t : S[cu]) {
          if (t.stage != st || t.layer != l) continue;
          if (t.type == TT_FIN) {
            if (!T.ks || t.nks != T.S || t.part_slot != part_base[st] * 4 || t.nsub < 1 || t.row0 % 16 ||
                t.row0 / 16 + t.nsub > nst || t.nchunks != 0)
              return MK_ERR_PLAN;
            for (int u = t.row0 / 16; u < t.row0 / 16 + t.nsub; ++u) fins[u] += 1;
            continue;
          }
          if (t.type != TT_GEMV) continue;
          if (t.row0 % 16 || t.nsub < 1 || t.nsub > 4 * tpw || t.row0 / 16 + t.nsub > nst) return MK_ERR_PLAN;
          if (t.k0 % kKBlock || t.k1 <= t.k0 || t.k1 > K) return MK_ERR_PLAN;
          if (t.nchunks != t.nsub * ((t.k1 - t.k0 + kKBlock - 1) / kKBlock)) return MK_ERR_PLAN;
          if (T.owner && (t.nks != 1 || t.k0 != 0 || t.k1 != K)) return MK_ERR_PLAN;
          if (T.ks) {
            const int wkb = std::max(1, ((pc.xb_bytes / (4 * batch)) - 8) / kKBlock);
            if (!(t.flags & kTaskPublish) || t.nks != T.S || t.part_slot != part_base[st] * 4 ||
                (t.k1 - t.k0 + kKBlock - 1) / kKBlock > wkb || t.k0 != piece_kb(t.ks, T.nkb, T.S) * kKBlock)
              return MK_ERR_PLAN;
          } else if (!T.owner &&
                     (t.nsub > T.gs || t.row0 != t.group * 16 * T.gs || t.nks != group_pieces[st][t.group])) {
            return MK_ERR_PLAN;
          }
          for (int u = t.row0 / 16; u < t.row0 / 16 + t.nsub; ++u) {
            if (t.k0 != next_k[u] || t.ks != pieces[u]) return MK_ERR_PLAN;
            next_k[u] = t.k1;
            pieces[u] += 1;
          }
          covered += (long long)std::min(16 * t.nsub, M - t.row0) * (t.k1 - t.k0);
        }
      for (int u = 0; u < nst; ++u) {
        if (next_k[u] != K) return MK_ERR_PLAN;
        if (T.ks && (pieces[u] != T.S || fins[u] != 1)) return MK_ERR_PLAN;
        if (!T.owner && !T.ks && pieces[u] != group_pieces[st][u / T.gs]) return MK_ERR_PLAN;
      }
      if (covered != (long long)M * K) return MK_ERR_PLAN;
    }
  }
  // (2) deadlock freedom.  The device has three kinds of wait, each modelled
  //     here as a wait on ALL the tasks that could produce what it polls (a
  //     superset of its real producers, so a schedule that completes here
  //     cannot deadlock on the device):
  //       * a stage's inputs (step-tagged words of the previous stage's
  //         output): every task of that stage;
  //       * a split group's piece 0 (after its own piece), a K-split finish
  //         task: every piece of the stage in that layer;
  //       * attention's segment finisher (after the CU's own pieces): every
  //         attention piece of the layer (the partition is cut on the device).
  //     Each task is one or two phases (wait, signal); the in-order streams
  //     run abstractly until nothing can move.
  {
    const int kStages = 7;  // QKV ATTN O GU DOWN LM EMBED
    auto out_ctr = [&](int st, int l) { return 2 * (l * kStages + st); };
    auto piece_ctr = [&](int st, int l) { return 2 * (l * kStages + st) + 1; };
    auto prev_out = [&](int st, int l) {
      switch (st) {
        case ST_QKV: return l == 0 ? out_ctr(ST_EMBED, 0) : out_ctr(ST_DOWN, l - 1);
        case ST_ATTN: return out_ctr(ST_QKV, l);
        case ST_O: return out_ctr(ST_ATTN, l);
        case ST_GU: return out_ctr(ST_O, l);
        case ST_DOWN: return out_ctr(ST_GU, l);
        case ST_LM: return out_ctr(ST_DOWN, pc.L - 1);
      }
      return -1;
    };
    struct Ph {
      int wait, signal;
    };
    const int nctr = 2 * (pc.L + 1) * kStages;
    std::vector<std::vector<Ph>> prog(ncu);
    std::vector<int> total(nctr, 0), given(nctr, 0);
    for (int c = 0; c < ncu; ++c)
      for (const Task& t : S[c]) {
        const int l = t.layer;
        if (t.type == TT_EMBED) {
          prog[c].push_back({-1, out_ctr(ST_EMBED, 0)});
        } else if (t.type == TT_ATTN) {
          prog[c].push_back({prev_out(ST_ATTN, l), piece_ctr(ST_ATTN, l)});
          prog[c].push_back({piece_ctr(ST_ATTN, l), out_ctr(ST_ATTN, l)});
        } else if (t.type == TT_FIN) {
          prog[c].push_back({piece_ctr(t.stage, l), out_ctr(t.stage, l)});
        } else if (t.flags & kTaskPublish) {
          prog[c].push_back({prev_out(t.stage, l), piece_ctr(t.stage, l)});
        } else if (t.nks > 1) {
          prog[c].push_back({prev_out(t.stage, l), piece_ctr(t.stage, l)});
          if (t.ks == 0) prog[c].push_back({piece_ctr(t.stage, l), out_ctr(t.stage, l)});
        } else {
          prog[c].push_back({prev_out(t.stage, l), out_ctr(t.stage, l)});
        }
      }
    size_t nph = 0;
    for (int c = 0; c < ncu; ++c)
      for (const Ph& ph : prog[c]) {
        total[ph.signal] += 1;
        nph += 1;
      }
    std::vector<size_t> pcx(ncu, 0);
    size_t done = 0;
    bool progress = true;
    while (progress) {
      progress = false;
      for (int c = 0; c < ncu; ++c) {
        while (pcx[c] < prog[c].size()) {
          const Ph& ph = prog[c][pcx[c]];
          if (ph.wait >= 0 && (total[ph.wait] == 0 || given[ph.wait] < total[ph.wait])) break;
          given[ph.signal] += 1;
          pcx[c] += 1;
          done += 1;
          progress = true;
        }
      }
    }
    if (done != nph) return MK_ERR_PLAN;
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
  P.attn_map = (int*)malloc(sizeof(int) * attn_map.size());
  if (!P.tasks || !P.task_off || !P.expect || !P.attn_map) {
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
  memcpy(P.attn_map, attn_map.data(), sizeof(int) * attn_map.size());
  *out = P;
  return MK_OK;
}

}  // namespace mk
