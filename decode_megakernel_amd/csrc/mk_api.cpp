// C ABI of the decode-step megakernel: argument checks, workspace, schedule
// cache and the single launch per step.  See include/mk.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {
hipError_t launch_step(const DevArgs& A, hipStream_t stream, bool coop);
hipError_t step_occupancy(size_t lds, int* blocks_per_cu);
hipError_t static_scratch_base(void** out);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_untag_copy(void* dst, size_t dpitch, const void* src, size_t spitch, size_t row_bytes, size_t rows,
                             hipStream_t stream);
size_t lds_bytes(int nslot, int xb_bytes);
}  // namespace mk

using namespace mk;

namespace {

struct GraphDev {
  Plan plan;
  int nslot = 0;  // LDS ring slots of this batch size's launches
  int xb = 0;     // LDS bytes left to stage GEMV inputs
  Task* d_tasks = nullptr;
  int* d_off = nullptr;
  int* d_expect = nullptr;
  int* d_attn_map = nullptr;
};

int env_int(const char* name, int def) {
  const char* v = getenv(name);
  if (!v || !*v) return def;
  return atoi(v);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct mk_handle {
  mk_model_cfg cfg;
  int device = 0;
  int ncu = 0;
  int nslot = 7;    // ring slots with no batch rule applied (the smallest staging buffer)
  int xb = 0;
  int lds_max = 0;  // LDS bytes per work-group
  int mfma_min_batch = 8;
  uint64_t timeout_ticks = 0;
  LayerW* d_layers = nullptr;
  const uint16_t* embed = nullptr;
  const uint16_t* lm_head = nullptr;
  const uint16_t* final_norm = nullptr;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  size_t tagged_bytes = 0;  // leading workspace bytes whose words carry step tags
  uint32_t rowtag = 0;      // bit n: the step tag sequence n's words carry now
  // workspace views
  float *hres, *hmid, *ssattn, *ssmlp, *qkv, *apart, *rope, *zero;
  float *xattn, *xmlp, *attn_out, *act;
  uint32_t *banks, *status;
  int ctr_stride = 0, bank_words = 0;
  std::map<int, GraphDev> graphs;  // one schedule per batch size 1..max_batch, built by mk_create
  float* d_part = nullptr;          // split-K partial slots, shared by every schedule (all zero between steps)
  size_t part_bytes = 0;
  int coop = 1;                     // cooperative launches (co-residency guaranteed by the runtime)
  float* dump = nullptr;            // caller's mid-state dump buffer (mk_set_midstate_dump), NULL = off
  // workspace offsets: the allocation-free step lays the same buffers out in
  // the static scratch array (activations and partials from offset 0, the
  // counter banks at o_banks, the split-K slots at o_part)
  size_t o_hres = 0, o_hmid = 0, o_xattn = 0, o_xmlp = 0, o_ssattn = 0, o_ssmlp = 0, o_qkv = 0, o_aout = 0,
         o_act = 0, o_apart = 0, o_banks = 0, o_part = 0, static_bytes = 0;
  void* sbase = nullptr;            // this device's static scratch array (looked up at mk_create)
  uint64_t step = 0;
  uint64_t* trace = nullptr;   // MK_TRACE=<tasks per CU>: per-task timestamps + per-CU wait totals
  int trace_cap = 0;
  int attn_pad = 0;            // attention partition: empty rows ahead of each segment (upper bound)
  int attn_min_rows = 32;      // attention partition: rows a CU takes at least
  int ctx_bound = 0;           // caller's bound on seq_lens (mk_set_context_bound), 0 = none
  bool knob_pad = false, knob_min_rows = false;  // partition fixed from the environment
};

extern "C" {

const char* mk_error_string(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "unsupported model shape";
    case MK_ERR_OOM: return "device out of memory";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_PLAN: return "schedule validation failed";
    case MK_ERR_TOO_LARGE: return "the step's scratch exceeds the static scratch array (64 MiB per GPU)";
  }
  return "unknown error";
}

static int build_graph(mk_handle* h, int b);
static size_t part_bytes_of(const mk_handle* h, const GraphDev& g);

static int check_cfg(const mk_model_cfg* c) {
  if (!c) return MK_ERR_INVALID_ARG;
  if (c->n_layers < 1 || c->hidden < 64 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->intermediate < 64 ||
      c->vocab < 1 || c->max_batch < 1 || c->max_batch > kMaxBatch || c->max_seq < 1 || !(c->rms_eps > 0.f) ||
      !(c->rope_theta > 0.0))
    return MK_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads) return MK_ERR_INVALID_ARG;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->head_dim != 64 && c->head_dim != 128) return MK_ERR_UNSUPPORTED;
  if (G > (c->head_dim == 128 ? 4 : 8)) return MK_ERR_UNSUPPORTED;
  if (c->hidden % 64 || c->intermediate % 64) return MK_ERR_UNSUPPORTED;
  // the input staging sums at most 512 per-16-row partial sums of squares
  if (c->hidden > 8192) return MK_ERR_UNSUPPORTED;
  // attention's flattened (sequence, KV head, position) rows are counted in 32 bits
  if ((long long)c->n_kv_heads * c->max_batch * c->max_seq >= (1LL << 31)) return MK_ERR_UNSUPPORTED;
  // a K slice of one row of 16 bf16 columns per sequence must fit the staging buffer
  return MK_OK;
}

static PlanCfg plan_cfg(const mk_model_cfg* c, int ncu, int xb, int mfma_min) {
  PlanCfg p;
  p.L = c->n_layers;
  p.d = c->hidden;
  p.nq = c->n_q_heads;
  p.nkv = c->n_kv_heads;
  p.hd = c->head_dim;
  p.I = c->intermediate;
  p.V = c->vocab;
  p.ncu = ncu;
  p.xb_bytes = xb;
  p.mfma_min_batch = mfma_min;
  p.gemv_mode = env_int("MK_GEMV_MODE", 0);
  p.skip_prev = env_int("MK_PLAN_SKIP_PREV", 2);
  p.attn_idle = env_int("MK_ATTN_IDLE", 1);
  p.ksplit = env_int("MK_KSPLIT", 1);
  p.window_chunks = env_int("MK_WINDOW_COST", 6);
  p.split_chunks = env_int("MK_SPLIT_COST", 6);
  p.ksplit_aligned = env_int("MK_KSPLIT_ALIGNED", 1);
  // MK_GEMV_STAGE_MODES="qkv:2,o:3,...": the tiling of single stages (1 row-owner,
  // 2 stream-K, 3 stream-K with one-tile groups)
  if (const char* v = getenv("MK_GEMV_STAGE_MODES")) {
    const char* names[6] = {"qkv", "", "o", "gu", "down", "lm"};
    for (int st = 0; st < 6; ++st) {
      if (!names[st][0]) continue;
      char key[8];
      snprintf(key, sizeof key, "%s:", names[st]);
      const char* f = strstr(v, key);
      if (f && (f == v || f[-1] == ',')) p.stage_mode[st] = atoi(f + strlen(key));
    }
  }
  p.ksplit_min_windows = env_int("MK_KSPLIT_MIN_WINDOWS", 4);
  return p;
}

static int xb_for(int lds_max, int nslot) {
  long long xb = (long long)lds_max - (long long)nslot * kSlotBytes - kRedBytes - kCtrlBytes;
  xb &= ~255LL;
  return (int)xb;
}

// Ring slots for a batch: 7 by default.  An MFMA batch (>= mfma_min) whose
// GEMV input windows (K blocks staged at once, 4 bytes per element and
// sequence) grow when one slot's 16 KB goes to the staging buffer takes 6:
// fewer restaging round trips outweigh the shallower prefetch (Llama-3-8B
// b9 7.29 -> 7.12 ms; at batch 16 the window stays one block and 6 slots are
// slower).  MK_NSLOT, when set, fixes the count for every batch.
static int nslot_for(int lds_max, int b, int mfma_min) {
  const char* v = getenv("MK_NSLOT");
  int n = (v && *v) ? atoi(v) : 7;
  if (!(v && *v) && b >= mfma_min) {
    auto wkb = [&](int nslot) { return std::max(1, ((xb_for(lds_max, nslot) / (4 * b)) - 8) / kKBlock); };
    if (wkb(6) > wkb(7)) n = 6;
  }
  // a loader wave publishes a chunk only after issuing its next one, so the
  // ring must hold more chunks than there are loader waves
  return std::min(kMaxSlots, std::max(kLoaderWaves + 1, n));
}

int mk_plan(const mk_model_cfg* cfg, int32_t batch, int32_t n_cu, mk_plan_stats* out) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!out || n_cu < 1 || batch < 1 || batch > cfg->max_batch) return MK_ERR_INVALID_ARG;
  const int mfma_min = std::min(8, std::max(1, env_int("MK_MFMA_MIN_BATCH", 8)));
  PlanCfg pc = plan_cfg(cfg, n_cu, xb_for(163840, nslot_for(163840, batch, mfma_min)), mfma_min);
  Plan P;
  rc = build_plan(pc, batch, &P);
  if (rc) return rc;
  memset(out, 0, sizeof(*out));
  out->n_tasks = P.n_tasks;
  out->max_tasks_per_cu = P.max_tasks_per_cu;
  out->n_counters = P.n_counters;
  out->mfma = P.mfma;
  out->weight_bytes = P.weight_bytes;
  out->max_cu_weight_bytes = P.max_cu_weight_bytes;
  out->stage_balance_min = P.balance_min;
  for (int i = 0; i < 6; ++i) {
    out->stage_tasks[i] = P.stage_tasks[i];
    out->stage_ksplit[i] = P.stage_ksplit[i];
    out->stage_rows_per_task[i] = P.stage_rows[i];
    out->stage_kpieces[i] = P.stage_kpieces[i];
  }
  // placement of one layer: which CUs run each stage
  {
    const int L = cfg->n_layers, lay = L > 1 ? 1 : 0;
    auto cus_of = [&](int stage, int layer) {
      std::vector<char> u(n_cu, 0);
      for (int c = 0; c < n_cu; ++c)
        for (int k = P.task_off[c]; k < P.task_off[c + 1]; ++k)
          if (P.tasks[k].stage == stage && P.tasks[k].layer == layer && P.tasks[k].type == TT_GEMV) u[c] = 1;
      return u;
    };
    const int* m = P.attn_map + (size_t)lay * (n_cu + 1);
    std::vector<char> attn(n_cu, 1);
    if (m[n_cu] > 0)
      for (int c = 0; c < n_cu; ++c) attn[c] = m[c] < m[n_cu];
    std::vector<char> sets[6] = {cus_of(ST_QKV, lay), attn, cus_of(ST_O, lay), cus_of(ST_GU, lay),
                                 cus_of(ST_DOWN, lay), cus_of(ST_LM, L)};
    std::vector<char> prev[6] = {lay > 0 ? cus_of(ST_DOWN, lay - 1) : std::vector<char>(n_cu, 0), sets[0], sets[1],
                                 sets[2], sets[3], cus_of(ST_DOWN, L - 1)};
    for (int i = 0; i < 6; ++i)
      for (int c = 0; c < n_cu; ++c) {
        out->stage_cus[i] += sets[i][c];
        out->stage_shared_prev[i] += sets[i][c] && prev[i][c];
      }
    out->attn_slot_cap = m[n_cu];
    int valid = 1;
    for (int l = 0; l < L && valid; ++l) {
      std::vector<char> seen(n_cu, 0);
      for (int c = 0; c < n_cu; ++c) {
        const int v = P.attn_map[(size_t)l * (n_cu + 1) + c];
        if (v < 0 || v >= n_cu || seen[v]) valid = 0;
        else seen[v] = 1;
      }
    }
    out->attn_slots_valid = valid;
  }
  free_plan(&P);
  return MK_OK;
}

int mk_plan_streams(const mk_model_cfg* cfg, int32_t batch, int32_t n_cu, mk_task_info* tasks, int32_t cap,
                    int32_t* cu_offsets, int32_t* attn_map, int32_t* n_tasks) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!n_tasks || !cu_offsets || n_cu < 1 || batch < 1 || batch > cfg->max_batch || cap < 0)
    return MK_ERR_INVALID_ARG;
  const int mfma_min = std::min(8, std::max(1, env_int("MK_MFMA_MIN_BATCH", 8)));
  PlanCfg pc = plan_cfg(cfg, n_cu, xb_for(163840, nslot_for(163840, batch, mfma_min)), mfma_min);
  Plan P;
  rc = build_plan(pc, batch, &P);
  if (rc) return rc;
  *n_tasks = P.n_tasks;
  if (P.n_tasks > cap || !tasks) {
    free_plan(&P);
    return MK_ERR_INVALID_ARG;
  }
  for (int i = 0; i < P.n_tasks; ++i) {
    const Task& t = P.tasks[i];
    mk_task_info& o = tasks[i];
    o.type = t.type;
    o.stage = t.stage;
    o.layer = t.layer;
    o.row0 = t.row0;
    o.nsub = t.nsub;
    o.k0 = t.k0;
    o.k1 = t.k1;
    o.ks = t.ks;
    o.nks = t.nks;
    o.group = t.group;
    o.part_slot = t.part_slot;
    o.nchunks = t.nchunks;
    o.flags = t.flags;
  }
  for (int c = 0; c <= n_cu; ++c) cu_offsets[c] = P.task_off[c];
  if (attn_map) memcpy(attn_map, P.attn_map, sizeof(int) * (size_t)cfg->n_layers * (n_cu + 1));
  free_plan(&P);
  return MK_OK;
}

int mk_create(const mk_model_cfg* cfg, const mk_weight_ptrs* w, mk_handle** out) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!w || !out) return MK_ERR_INVALID_ARG;
  const int L = cfg->n_layers;
  if (!w->embed || !w->final_norm || (!cfg->tied_embeddings && !w->lm_head) || !w->attn_norm || !w->q_proj ||
      !w->k_proj || !w->v_proj || !w->o_proj || !w->mlp_norm || !w->gate_proj || !w->up_proj || !w->down_proj)
    return MK_ERR_INVALID_ARG;
  if (cfg->qk_norm && (!w->q_norm || !w->k_norm)) return MK_ERR_INVALID_ARG;
  for (int l = 0; l < L; ++l) {
    if (!w->attn_norm[l] || !w->q_proj[l] || !w->k_proj[l] || !w->v_proj[l] || !w->o_proj[l] || !w->mlp_norm[l] ||
        !w->gate_proj[l] || !w->up_proj[l] || !w->down_proj[l])
      return MK_ERR_INVALID_ARG;
    if (cfg->qk_norm && (!w->q_norm[l] || !w->k_norm[l])) return MK_ERR_INVALID_ARG;
  }
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return MK_ERR_OOM;
  h->cfg = *cfg;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return MK_ERR_HIP;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) != hipSuccess) {
    delete h;
    return MK_ERR_HIP;
  }
  h->ncu = env_int("MK_NUM_CU", prop.multiProcessorCount);
  if (h->ncu < 1 || h->ncu > prop.multiProcessorCount) h->ncu = prop.multiProcessorCount;
  h->lds_max = (int)prop.sharedMemPerBlock;
  // the smallest staging buffer any batch gets (the most ring slots)
  h->nslot = std::max(nslot_for(h->lds_max, 1, 1 << 30), nslot_for(h->lds_max, cfg->max_batch, 1 << 30));
  h->xb = xb_for(h->lds_max, h->nslot);
  // the staging buffer holds attention's softmax states, and one 512-wide K
  // block of every sequence's input as bf16 hi + lo halves (plus padding)
  if (h->xb < kAttnStateBytes || h->xb < cfg->max_batch * (kKBlock + 8) * 4) {
    delete h;
    return MK_ERR_UNSUPPORTED;
  }
  // the VALU path handles up to 7 sequences; larger batches use MFMA tiles
  h->mfma_min_batch = std::min(8, std::max(1, env_int("MK_MFMA_MIN_BATCH", 8)));
  h->timeout_ticks = (uint64_t)env_int("MK_SPIN_TIMEOUT_MS", 2000) * 100000ull;

  const int d = cfg->hidden, bc = cfg->max_batch, hd = cfg->head_dim, nkv = cfg->n_kv_heads;
  const int qdim = cfg->n_q_heads * hd, nqkv = qdim + 2 * nkv * hd, I = cfg->intermediate;
  h->ctr_stride = ctr_stride(L);
  h->bank_words = kShards * h->ctr_stride + 2 * kMaxBatch;
  // workspace layout
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  size_t o_hres = take((size_t)(L + 1) * bc * d * 4);
  size_t o_hmid = take((size_t)L * bc * d * 4);
  size_t o_xattn = take((size_t)(L + 1) * bc * d * 4);
  size_t o_xmlp = take((size_t)L * bc * d * 4);
  size_t o_ssattn = take((size_t)(L + 1) * (d / 16) * bc * 4);
  size_t o_ssmlp = take((size_t)L * (d / 16) * bc * 4);
  size_t o_qkv = take((size_t)L * bc * nqkv * 4);
  size_t o_aout = take((size_t)L * bc * qdim * 4);
  size_t o_act = take((size_t)L * bc * I * 4);
  // attention partial slots, per layer: [L][ncu + bc*nkv][group slots][hd + 4]
  const int G = cfg->n_q_heads / nkv, gm = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  size_t o_apart = take((size_t)L * (h->ncu + bc * nkv) * gm * (hd + 4) * 4);
  size_t o_banks = take((size_t)2 * h->bank_words * 4);
  size_t o_status = take(64);
  size_t o_rope = take((size_t)cfg->max_seq * (hd / 2) * 2 * 4);
  size_t o_zero = take(1024);
  h->ws_bytes = off;
  h->tagged_bytes = o_banks;  // hres .. apart: words that carry step tags / validity flags
  h->o_hres = o_hres;
  h->o_hmid = o_hmid;
  h->o_xattn = o_xattn;
  h->o_xmlp = o_xmlp;
  h->o_ssattn = o_ssattn;
  h->o_ssmlp = o_ssmlp;
  h->o_qkv = o_qkv;
  h->o_aout = o_aout;
  h->o_act = o_act;
  h->o_apart = o_apart;
  h->o_banks = o_banks;
  h->o_part = o_status;  // the banks end here
  if (hipMalloc(&h->ws, h->ws_bytes) != hipSuccess) {
    delete h;
    return MK_ERR_OOM;
  }
  if (hipMemset(h->ws, 0, h->ws_bytes) != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    return MK_ERR_HIP;
  }
  h->hres = (float*)(h->ws + o_hres);
  h->hmid = (float*)(h->ws + o_hmid);
  h->xattn = (float*)(h->ws + o_xattn);
  h->xmlp = (float*)(h->ws + o_xmlp);
  h->ssattn = (float*)(h->ws + o_ssattn);
  h->ssmlp = (float*)(h->ws + o_ssmlp);
  h->qkv = (float*)(h->ws + o_qkv);
  h->attn_out = (float*)(h->ws + o_aout);
  h->act = (float*)(h->ws + o_act);
  h->apart = (float*)(h->ws + o_apart);
  h->banks = (uint32_t*)(h->ws + o_banks);
  h->status = (uint32_t*)(h->ws + o_status);
  h->rope = (float*)(h->ws + o_rope);
  h->zero = (float*)(h->ws + o_zero);

  // RoPE table: angle p * theta^(-2j/hd), computed in double on the host.
  {
    std::vector<float> t((size_t)cfg->max_seq * (hd / 2) * 2);
    for (int p = 0; p < cfg->max_seq; ++p)
      for (int j = 0; j < hd / 2; ++j) {
        double a = (double)p * std::pow(cfg->rope_theta, -2.0 * j / hd);
        t[((size_t)p * (hd / 2) + j) * 2] = (float)std::cos(a);
        t[((size_t)p * (hd / 2) + j) * 2 + 1] = (float)std::sin(a);
      }
    if (hipMemcpy(h->rope, t.data(), t.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(h->ws);
      delete h;
      return MK_ERR_HIP;
    }
  }
  // per-layer weight pointers
  {
    std::vector<LayerW> lw(L);
    for (int l = 0; l < L; ++l) {
      lw[l].attn_norm = (const uint16_t*)w->attn_norm[l];
      lw[l].q = (const uint16_t*)w->q_proj[l];
      lw[l].k = (const uint16_t*)w->k_proj[l];
      lw[l].v = (const uint16_t*)w->v_proj[l];
      lw[l].o = (const uint16_t*)w->o_proj[l];
      lw[l].q_norm = cfg->qk_norm ? (const uint16_t*)w->q_norm[l] : nullptr;
      lw[l].k_norm = cfg->qk_norm ? (const uint16_t*)w->k_norm[l] : nullptr;
      lw[l].mlp_norm = (const uint16_t*)w->mlp_norm[l];
      lw[l].gate = (const uint16_t*)w->gate_proj[l];
      lw[l].up = (const uint16_t*)w->up_proj[l];
      lw[l].down = (const uint16_t*)w->down_proj[l];
    }
    if (hipMalloc(&h->d_layers, sizeof(LayerW) * L) != hipSuccess) {
      (void)hipFree(h->ws);
      delete h;
      return MK_ERR_OOM;
    }
    if (hipMemcpy(h->d_layers, lw.data(), sizeof(LayerW) * L, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(h->d_layers);
      (void)hipFree(h->ws);
      delete h;
      return MK_ERR_HIP;
    }
  }
  // A CU whose attention rows cross into a new segment runs a second piece
  // (query load, wave merge, partial publish) and usually finishes that
  // segment: padding each segment's start charges it about 256 KB of K/V
  // rows' worth of time (512 rows at head_dim 128; the kernel caps the pad
  // at half a CU's rows).
  h->attn_pad = std::max(0, env_int("MK_ATTN_PAD", (256 << 10) / (4 * cfg->head_dim)));
  h->attn_min_rows = std::max(1, env_int("MK_ATTN_MIN_ROWS", 32));
  h->knob_pad = getenv("MK_ATTN_PAD") && *getenv("MK_ATTN_PAD");
  h->knob_min_rows = getenv("MK_ATTN_MIN_ROWS") && *getenv("MK_ATTN_MIN_ROWS");
  h->trace_cap = env_int("MK_TRACE", 0);
  if (h->trace_cap > 0) {
    size_t tb = ((size_t)h->ncu * h->trace_cap * 4 + (size_t)h->ncu * kStatWords) * 8;
    if (hipMalloc(&h->trace, tb) != hipSuccess || hipMemset(h->trace, 0, tb) != hipSuccess) {
      (void)hipFree(h->d_layers);
      (void)hipFree(h->ws);
      delete h;
      return MK_ERR_OOM;
    }
  }
  h->embed = (const uint16_t*)w->embed;
  h->lm_head = cfg->tied_embeddings ? (const uint16_t*)w->embed : (const uint16_t*)w->lm_head;
  h->final_norm = (const uint16_t*)w->final_norm;
  // every schedule the handle can run (batch 1..max_batch) is built, validated
  // and uploaded here, so a step never allocates, copies or synchronises on
  // the host (a new batch size mid-run is a lookup)
  for (int b = 1; b <= cfg->max_batch; ++b) {
    rc = build_graph(h, b);
    if (rc) {
      mk_destroy(h);
      return rc;
    }
  }
  // the persistent work-groups poll one another: check that one of them fits
  // a CU with the largest LDS any schedule asks for
  size_t lds_need = 0;
  for (auto& kv : h->graphs) {
    lds_need = std::max(lds_need, lds_bytes(kv.second.nslot, kv.second.xb));
    h->part_bytes = std::max(h->part_bytes, part_bytes_of(h, kv.second));
  }
  int per_cu = 0;
  if (step_occupancy(lds_need, &per_cu) != hipSuccess || per_cu < 1) {
    mk_destroy(h);
    return MK_ERR_UNSUPPORTED;
  }
  if (hipMalloc(&h->d_part, h->part_bytes) != hipSuccess) {
    mk_destroy(h);
    return MK_ERR_OOM;
  }
  if (hipMemset(h->d_part, 0, h->part_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    mk_destroy(h);
    return MK_ERR_HIP;
  }
  // set-up of the allocation-free step: this device's static scratch array
  h->static_bytes = h->o_part + h->part_bytes;
  if (static_scratch_base(&h->sbase) != hipSuccess) {
    mk_destroy(h);
    return MK_ERR_HIP;
  }
  int coop_ok = 0;
  if (hipDeviceGetAttribute(&coop_ok, hipDeviceAttributeCooperativeLaunch, h->device) != hipSuccess) coop_ok = 0;
  h->coop = coop_ok && env_int("MK_COOP", 1) != 0;
  *out = h;
  return MK_OK;
}

static void free_graph(GraphDev& g) {
  (void)hipFree(g.d_tasks);
  (void)hipFree(g.d_off);
  (void)hipFree(g.d_expect);
  (void)hipFree(g.d_attn_map);
  free_plan(&g.plan);
}

// Build, validate and upload the schedule of batch size b (mk_create only:
// the step never allocates or copies on the host side).
static int build_graph(mk_handle* h, int b) {
  GraphDev g;
  g.nslot = nslot_for(h->lds_max, b, h->mfma_min_batch);
  g.xb = xb_for(h->lds_max, g.nslot);
  PlanCfg pc = plan_cfg(&h->cfg, h->ncu, g.xb, h->mfma_min_batch);
  int rc = build_plan(pc, b, &g.plan);
  if (rc) return rc;
  const Plan& P = g.plan;
  bool ok = hipMalloc(&g.d_tasks, sizeof(Task) * (size_t)std::max(1, P.n_tasks)) == hipSuccess &&
            hipMalloc(&g.d_off, sizeof(int) * (h->ncu + 1)) == hipSuccess &&
            hipMalloc(&g.d_expect, sizeof(int) * (size_t)P.n_counters * kShards) == hipSuccess &&
            hipMalloc(&g.d_attn_map, sizeof(int) * (size_t)pc.L * (h->ncu + 1)) == hipSuccess;
  if (!ok) {
    free_graph(g);
    return MK_ERR_OOM;
  }
  ok = hipMemcpy(g.d_tasks, P.tasks, sizeof(Task) * P.n_tasks, hipMemcpyHostToDevice) == hipSuccess &&
       hipMemcpy(g.d_off, P.task_off, sizeof(int) * (h->ncu + 1), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemcpy(g.d_expect, P.expect, sizeof(int) * (size_t)P.n_counters * kShards, hipMemcpyHostToDevice) == hipSuccess &&
       hipMemcpy(g.d_attn_map, P.attn_map, sizeof(int) * (size_t)pc.L * (h->ncu + 1), hipMemcpyHostToDevice) == hipSuccess;
  if (!ok) {
    free_graph(g);
    return MK_ERR_HIP;
  }
  h->graphs.emplace(b, g);
  return MK_OK;
}

static size_t part_bytes_of(const mk_handle* h, const GraphDev& g) {
  return sizeof(float) * 1024 * (size_t)(h->cfg.n_layers + 1) * std::max(1, g.plan.part_blocks);
}

// Checks and kernel arguments shared by both step entry points; the
// workspace pointers are the handle's own.
// The KV cache of a step: contiguous rows per sequence, or paged blocks.
struct KVDesc {
  void *k = nullptr, *v = nullptr;
  int bcap = 0, scap = 0;            // contiguous: sequence rows and positions per row
  const int32_t* btab = nullptr;     // paged: block table, NULL for contiguous
  int bt_stride = 0, bsize = 0, nblocks = 0;
};

// Context routing: with a context bound declared by the caller, the attention
// partition of a step takes the parameters measured best for its (batch
// class, context bucket) on a Qwen3-8B-shaped model (head_dim 128, 8 KV
// heads) swept over contexts 64-4096: (empty rows ahead of each segment in
// units of 256 KB of K/V rows, rows a CU takes at least).  Without a bound
// (or with the partition fixed from the environment) the defaults apply.
static void route_attention(const mk_handle* h, int batch, DevArgs& A) {
  if (h->ctx_bound <= 0) return;
  struct Route {
    int max_ctx;
    int pad_quarters;  // pad = pad_quarters / 4 x 256 KB of K/V rows
    int min_rows;
  };
  static const Route small_b[] = {{128, 4, 128}, {512, 1, 8}, {2048, 0, 8}, {1 << 30, 0, 32}};
  static const Route large_b[] = {{128, 4, 8}, {512, 4, 32}, {2048, 0, 128}, {1 << 30, 0, 128}};
  const Route* tab = batch >= 8 ? large_b : small_b;
  int k = 0;
  while (h->ctx_bound > tab[k].max_ctx) ++k;
  if (!h->knob_pad) A.attn_pad = tab[k].pad_quarters * ((256 << 10) / (4 * h->cfg.head_dim)) / 4;
  if (!h->knob_min_rows) A.attn_min_rows = tab[k].min_rows;
}

static int step_args(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                     const int32_t* seq_lens, const KVDesc* kv, float* logits_out, int32_t* next_tokens_out,
                     DevArgs& A, GraphDev** gout) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (batch < 0 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
  if (batch == 0) return MK_OK;
  if (!tokens || !positions || !seq_lens || !kv || !kv->k || !kv->v || !logits_out) return MK_ERR_INVALID_ARG;
  if (kv->btab) {
    // a chunk of cached rows (at most 64) must span at most two blocks
    if (kv->bsize < 64 || kv->nblocks < 1 || kv->bt_stride < 1) return MK_ERR_INVALID_ARG;
  } else if (kv->bcap < batch || kv->scap < 1) {
    return MK_ERR_INVALID_ARG;
  }
  if ((long long)h->cfg.n_kv_heads * batch * kv->scap >= (1LL << 31)) return MK_ERR_UNSUPPORTED;
  auto git = h->graphs.find(batch);
  if (git == h->graphs.end()) return MK_ERR_INVALID_ARG;  // every batch 1..max_batch is built by mk_create
  GraphDev* g = &git->second;
  *gout = g;
  const mk_model_cfg& c = h->cfg;
  memset(&A, 0, sizeof(A));
  A.L = c.n_layers;
  A.d = c.hidden;
  A.nq = c.n_q_heads;
  A.nkv = c.n_kv_heads;
  A.hd = c.head_dim;
  A.G = c.n_q_heads / c.n_kv_heads;
  A.I = c.intermediate;
  A.V = c.vocab;
  A.qdim = c.n_q_heads * c.head_dim;
  A.kvdim = c.n_kv_heads * c.head_dim;
  A.nqkv = A.qdim + 2 * A.kvdim;
  A.qk_norm = c.qk_norm;
  A.max_seq = c.max_seq;
  A.eps = c.rms_eps;
  A.layers = h->d_layers;
  A.embed = h->embed;
  A.lm_head = h->lm_head;
  A.final_norm = h->final_norm;
  A.kc = (uint16_t*)kv->k;
  A.vc = (uint16_t*)kv->v;
  A.kv_bcap = kv->bcap;
  A.kv_scap = kv->scap;
  A.btab = kv->btab;
  A.bt_stride = kv->bt_stride;
  A.bsize = kv->bsize;
  A.nblocks = kv->nblocks;
  A.tokens = tokens;
  A.positions = positions;
  A.seq_lens = seq_lens;
  A.logits = logits_out;
  A.next_tokens = next_tokens_out;
  A.b = batch;
  A.bank = (int)(h->step & 1);
  // the sequences of this step flip their tag: words left by any earlier
  // step carry the old value
  A.rowtag = h->rowtag ^ ((1u << batch) - 1u);
  A.bcap = c.max_batch;
  A.hres = h->hres;
  A.hmid = h->hmid;
  A.xattn = h->xattn;
  A.xmlp = h->xmlp;
  A.ssattn = h->ssattn;
  A.ssmlp = h->ssmlp;
  A.qkv = h->qkv;
  A.attn_out = h->attn_out;
  A.act = h->act;
  A.part = h->d_part;
  A.apart = h->apart;
  A.banks = h->banks;
  A.status = h->status;
  A.rope = h->rope;
  A.zero = (const uint16_t*)h->zero;
  A.tasks = g->d_tasks;
  A.task_off = g->d_off;
  A.expect = g->d_expect;
  A.attn_map = g->d_attn_map;
  A.ctr_stride = h->ctr_stride;
  A.bank_words = h->bank_words;
  A.part_blocks = std::max(1, g->plan.part_blocks);
  A.ncu = h->ncu;
  A.nslot = g->nslot;
  A.xb_bytes = g->xb;
  A.mfma = g->plan.mfma;
  A.timeout_ticks = h->timeout_ticks;
  A.trace = h->trace;
  A.trace_cap = h->trace_cap;
  A.attn_pad = h->attn_pad;
  A.attn_min_rows = h->attn_min_rows;
  route_attention(h, batch, A);
  A.dump = h->dump;
  return MK_OK;
}

static KVDesc contiguous(const mk_kv_cache* kv) {
  KVDesc d;
  if (kv) {
    d.k = kv->k;
    d.v = kv->v;
    d.bcap = kv->batch_cap;
    d.scap = kv->seq_cap;
  }
  return d;
}

int mk_decode_step(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                   const int32_t* seq_lens, const mk_kv_cache* kv, float* logits_out, int32_t* next_tokens_out,
                   void* stream) {
  DevArgs A;
  GraphDev* g = nullptr;
  const KVDesc d = contiguous(kv);
  int rc = step_args(h, batch, tokens, positions, seq_lens, kv ? &d : nullptr, logits_out, next_tokens_out, A, &g);
  if (rc || batch == 0) return rc;
  if (launch_step(A, (hipStream_t)stream, h->coop != 0) != hipSuccess) return MK_ERR_HIP;
  h->rowtag = A.rowtag;
  h->step += 1;
  return MK_OK;
}

int mk_decode_step_paged(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                         const int32_t* seq_lens, const mk_paged_kv* kv, float* logits_out, int32_t* next_tokens_out,
                         void* stream) {
  if (!kv || !kv->block_table) return MK_ERR_INVALID_ARG;
  KVDesc d;
  d.k = kv->k;
  d.v = kv->v;
  d.btab = kv->block_table;
  d.bt_stride = kv->max_blocks_per_seq;
  d.bsize = kv->block_size;
  d.nblocks = kv->n_blocks;
  d.scap = kv->max_blocks_per_seq * kv->block_size;  // positions a sequence can address
  DevArgs A;
  GraphDev* g = nullptr;
  int rc = step_args(h, batch, tokens, positions, seq_lens, &d, logits_out, next_tokens_out, A, &g);
  if (rc || batch == 0) return rc;
  if (launch_step(A, (hipStream_t)stream, h->coop != 0) != hipSuccess) return MK_ERR_HIP;
  h->rowtag = A.rowtag;
  h->step += 1;
  return MK_OK;
}

int mk_decode_step_static(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                          const int32_t* seq_lens, const mk_kv_cache* kv, float* logits_out,
                          int32_t* next_tokens_out, void* stream) {
  DevArgs A;
  GraphDev* g = nullptr;
  const KVDesc d = contiguous(kv);
  int rc = step_args(h, batch, tokens, positions, seq_lens, kv ? &d : nullptr, logits_out, next_tokens_out, A, &g);
  if (rc || batch == 0) return rc;
  if (h->static_bytes > kStaticScratchBytes) return MK_ERR_TOO_LARGE;
  if (!h->sbase) return MK_ERR_HIP;
  // the same buffers at the same offsets inside the static array, cleared on
  // the caller's stream first (it keeps the previous call's contents): every
  // activation word then carries tag 0, so this step's sequences use tag 1,
  // and every partial slot and counter starts at zero
  char* base = (char*)h->sbase;
  A.hres = (float*)(base + h->o_hres);
  A.hmid = (float*)(base + h->o_hmid);
  A.xattn = (float*)(base + h->o_xattn);
  A.xmlp = (float*)(base + h->o_xmlp);
  A.ssattn = (float*)(base + h->o_ssattn);
  A.ssmlp = (float*)(base + h->o_ssmlp);
  A.qkv = (float*)(base + h->o_qkv);
  A.attn_out = (float*)(base + h->o_aout);
  A.act = (float*)(base + h->o_act);
  A.apart = (float*)(base + h->o_apart);
  A.banks = (uint32_t*)(base + h->o_banks);
  A.part = (float*)(base + h->o_part);
  A.rowtag = (1u << batch) - 1u;
  A.bank = 0;
  A.trace = nullptr;
  A.trace_cap = 0;
  if (launch_zero(base, h->static_bytes, (hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  if (launch_step(A, (hipStream_t)stream, h->coop != 0) != hipSuccess) return MK_ERR_HIP;
  return MK_OK;
}

int mk_copy_hidden(mk_handle* h, int32_t batch, float* dst, void* stream) {
  if (!h || !dst || batch < 1 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
  const size_t row = (size_t)batch * h->cfg.hidden * 4;
  const size_t spitch = (size_t)h->cfg.max_batch * h->cfg.hidden * 4;
  // copied with the step-tag bit cleared (bf16-exact values come back exact)
  if (launch_untag_copy(dst, row, h->hres, spitch, row, h->cfg.n_layers + 1, (hipStream_t)stream) != hipSuccess)
    return MK_ERR_HIP;
  return MK_OK;
}

int mk_copy_state(mk_handle* h, int32_t which, int32_t batch, void* dst, void* stream) {
  if (!h || !dst || batch < 1 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
  const mk_model_cfg& c = h->cfg;
  const int qdim = c.n_q_heads * c.head_dim, nqkv = qdim + 2 * c.n_kv_heads * c.head_dim;
  const void* src = nullptr;
  size_t width = 0, esize = 4, layers = c.n_layers;
  switch (which) {
    case MK_STATE_HIDDEN: src = h->hres; width = c.hidden; layers = c.n_layers + 1; break;
    case MK_STATE_HMID: src = h->hmid; width = c.hidden; break;
    case MK_STATE_QKV: src = h->qkv; width = nqkv; break;
    case MK_STATE_ATTN: src = h->attn_out; width = qdim; esize = 4; break;
    case MK_STATE_ACT: src = h->act; width = c.intermediate; esize = 4; break;
    default: return MK_ERR_INVALID_ARG;
  }
  const size_t row = (size_t)batch * width * esize, spitch = (size_t)c.max_batch * width * esize;
  if (launch_untag_copy(dst, row, src, spitch, row, layers, (hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  return MK_OK;
}

int mk_copy_trace(mk_handle* h, void* dst, int64_t bytes, int32_t* n_cu, int32_t* cap, void* stream) {
  if (!h || !n_cu || !cap) return MK_ERR_INVALID_ARG;
  *n_cu = h->ncu;
  *cap = h->trace_cap;
  if (!h->trace || !dst) return MK_OK;
  const size_t tb = ((size_t)h->ncu * h->trace_cap * 4 + (size_t)h->ncu * kStatWords) * 8;
  if (bytes < (int64_t)tb) return MK_ERR_INVALID_ARG;
  if (hipMemcpyAsync(dst, h->trace, tb, hipMemcpyDeviceToDevice, (hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  return MK_OK;
}

int mk_get_status(mk_handle* h, void* stream, uint32_t* status) {
  if (!h || !status) return MK_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  uint32_t s[2];
  if (hipMemcpy(s, h->status, 8, hipMemcpyDeviceToHost) != hipSuccess) return MK_ERR_HIP;
  // word 1 is the kernel's sticky abort flag: once a wait timed out, every
  // later step gives up its long waits too, so TIMEOUT stays reported until
  // mk_reset clears the flag
  *status = s[0] | (s[1] ? MK_STATUS_TIMEOUT : 0u);
  if (s[0] && hipMemset(h->status, 0, 4) != hipSuccess) return MK_ERR_HIP;
  return MK_OK;
}

int mk_reset(mk_handle* h, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  // activations back to tag 0 everywhere, matching rowtag 0: an abandoned
  // step may have left some words with a new tag
  h->rowtag = 0;
  bool ok = hipMemset(h->ws, 0, h->tagged_bytes) == hipSuccess &&
            hipMemset(h->banks, 0, (size_t)2 * h->bank_words * 4) == hipSuccess &&
            hipMemset(h->status, 0, 8) == hipSuccess;
  ok = ok && hipMemset(h->d_part, 0, h->part_bytes) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  return ok ? MK_OK : MK_ERR_HIP;
}

int mk_set_context_bound(mk_handle* h, int32_t max_seq_len) {
  if (!h || max_seq_len < 0) return MK_ERR_INVALID_ARG;
  h->ctx_bound = max_seq_len;
  return MK_OK;
}

int mk_set_midstate_dump(mk_handle* h, float* hidden_out) {
  if (!h) return MK_ERR_INVALID_ARG;
  h->dump = hidden_out;
  return MK_OK;
}

int mk_destroy(mk_handle* h) {
  if (!h) return MK_ERR_INVALID_ARG;
  for (auto& kv : h->graphs) free_graph(kv.second);
  (void)hipFree(h->d_part);
  (void)hipFree(h->trace);
  (void)hipFree(h->d_layers);
  (void)hipFree(h->ws);
  delete h;
  return MK_OK;
}

}  // extern "C"
