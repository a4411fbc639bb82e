// Internal definitions shared by the host planner/runtime and the device kernel.
#pragma once
#include <stdint.h>

// Helpers used by both the host planner and the device kernel.
#if defined(__HIP__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

namespace mk {

// Work-group shape: compute waves wait on dependencies and do the math;
// loader waves stream weights and cached K/V rows into an LDS ring and never
// wait on a dependency counter.
constexpr int kComputeWaves = 4;
constexpr int kLoaderWaves = 3;
constexpr int kThreads = 64 * (kComputeWaves + kLoaderWaves);
constexpr int kComputeThreads = 64 * kComputeWaves;
constexpr int kChunkBytes = 16384;          // data of one streamed chunk (16 rows x 512 bf16, or 32/64 K+V rows)
constexpr int kWaveLoads = kChunkBytes / 1024;  // 16 B per lane x 64 lanes per wave-load
// LDS ring slot: a GEMV chunk's 16 weight rows sit kRowPitch bytes apart (1 KB
// of data + 16 B of padding), so the 16 rows an MFMA A operand reads at one
// K offset fall in different LDS banks while every row still arrives as one
// contiguous 1 KB load
constexpr int kRowPitch = 1040;
constexpr int kSlotBytes = 16 * kRowPitch;
constexpr int kMaxSlots = 8;
constexpr int kShards = 64;                  // dependency counters are sharded 64 ways
constexpr int kMaxBatch = 16;
constexpr int kMaxGroup = 8;                 // n_q / n_kv
constexpr int kKBlock = 512;                 // K elements per chunk (64 lanes x 8 for VALU, 16 MFMA k-steps)
constexpr int kGroupSub = 4;                 // 16-row sub-tiles per row group (one per compute wave)
// LDS for the GEMV tile reductions: one 16-row x 16-sequence fp32 tile per
// compute wave.  Attention keeps its per-wave softmax states in the GEMV
// input staging buffer instead (the two never run at once), which needs
// kAttnStateBytes of it.
constexpr int kRedBytes = 4 * 256 * 4;
// attention's use of the staging buffer: wave states (2 piece parities x
// 4 waves x group x (hd + 4) fp32), the scaled queries and new K / V rows of
// a batch of kAttnBatch pieces, per-wave transposed probabilities; largest
// over head_dim 64 / group 8 and head_dim 128 / group 4
constexpr int kAttnBatch = 4;
constexpr int attn_lds_floats(int hd, int gm) {
  // per wave: P as bf16 hi + lo, [rows per chunk][group padded to 4 or 8] each
  return 2 * 4 * gm * (hd + 4) + kAttnBatch * gm * hd + kAttnBatch * 2 * hd + 4 * (4096 / hd) * (gm <= 4 ? 4 : 8);
}
constexpr int kAttnStateBytes =
    4 * (attn_lds_floats(64, 8) > attn_lds_floats(128, 4) ? attn_lds_floats(64, 8) : attn_lds_floats(128, 4));
constexpr int kStatWords = 80;
// Scratch of the allocation-free step (mk_decode_step_static): one file-scope
// device array per GPU, held until the process ends.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;               // trace: per-CU phase totals (uint64 words)
#ifndef MK_PHASE_TRACE
#define MK_PHASE_TRACE 0
#endif
constexpr int kCtrlBytes = MK_PHASE_TRACE ? 1536 : 1024;             // LDS control block (ring flags, per-wave state, sequence inputs)

enum Stage : int32_t { ST_QKV = 0, ST_ATTN = 1, ST_O = 2, ST_GU = 3, ST_DOWN = 4, ST_LM = 5, ST_EMBED = 6 };
enum TaskType : int32_t { TT_EMBED = 1, TT_GEMV = 2, TT_ATTN = 3, TT_FIN = 4 };

// One instruction of a CU's stream (64 bytes).
struct Task {
  int32_t type;
  int32_t stage;
  int32_t layer;
  int32_t row0;        // GEMV / FIN: first logical output row; EMBED: first column
  int32_t nsub;        // GEMV: 16-row sub-tiles of the task (1..4*tiles_per_wave); EMBED: number of columns
  int32_t k0, k1;      // GEMV: K range, k0 a multiple of 512
  int32_t ks, nks;     // GEMV: this task's piece index among the nks pieces that split the group's K
  int32_t group;       // GEMV: row group (counter index within the stage when nks > 1)
  int32_t part_slot;   // GEMV nks > 1: partial block of piece 0 of the group (piece k at part_slot + k);
                       // K-split stage (GEMV publish / FIN): first 256-float tile slot of the stage,
                       // sub-tile u's piece k at part_slot + u * nks + k
  int32_t wait_ctr;    // dependency counter to wait on, -1 = none
  int32_t signal_ctr;  // counter this task signals when its outputs are complete
  int32_t nchunks;     // GEMV: LDS chunks streamed by the loader (nsub x k-blocks)
  int32_t flags;       // kTaskSignal: signal signal_ctr after this task (the CU's last task of the stage);
                       // kTaskPublish: K-split piece, publishes every owned sub-tile's partial tile
  int32_t pad;
};
static_assert(sizeof(Task) == 64, "Task must be 64 bytes");

// 16-row sub-tiles one compute wave accumulates at once in a GEMV task
// (registers: tiles x 16 rows x batch for the VALU path, 4 per tile for
// MFMA).  A task holds up to 4x this many sub-tiles; wave w owns sub-tiles
// w, w+4, ...
MK_HD constexpr int tiles_per_wave(int nb_valu) {
  return nb_valu <= 0 ? 8 : nb_valu <= 2 ? 2 : 1;
}
constexpr int kMaxTilesPerWave = 8;

// Counter indices: EMBED, then 5 per layer, then LM.
MK_HD inline int ctr_embed() { return 0; }
MK_HD inline int ctr_stage(int layer, int stage) { return 1 + 5 * layer + stage; }  // stage in QKV..DOWN
MK_HD inline int ctr_lm(int n_layers) { return 1 + 5 * n_layers; }
MK_HD inline int n_counters(int n_layers) { return 2 + 5 * n_layers; }
// shard k of counter c lives at word k * stride + c; stride >= 32 words keeps
// shards of one counter on different 128-byte lines.
MK_HD inline int ctr_stride(int n_layers) {
  int n = n_counters(n_layers);
  return n < 32 ? 32 : n;
}

struct LayerW {
  const uint16_t* attn_norm;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* q_norm;
  const uint16_t* k_norm;
  const uint16_t* mlp_norm;
  const uint16_t* gate;
  const uint16_t* up;
  const uint16_t* down;
};

// Kernel argument block (passed by value).
struct DevArgs {
  // model shape
  int32_t L, d, nq, nkv, hd, G, I, V, qdim, kvdim, nqkv;
  int32_t qk_norm, max_seq;
  float eps;
  // weights
  const LayerW* layers;
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  // caller buffers
  uint16_t* kc;
  uint16_t* vc;
  int32_t kv_bcap, kv_scap;
  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* seq_lens;
  float* logits;
  int32_t* next_tokens;
  int32_t b;
  int32_t bank;
  uint32_t rowtag;      // bit n: step tag of sequence n (flipped each step it runs)
  // workspace (library-owned)
  int32_t bcap;         // workspace batch capacity
  float* hres;          // [L+1][bcap][d]
  float* hmid;          // [L][bcap][d]
  float* xattn;         // [L+1][bcap][d]  h * norm weight: GEMV input of QKV / LM head
  float* xmlp;          // [L][bcap][d]    h_mid * norm weight: GEMV input of gate/up
  float* ssattn;        // [L+1][d/16][bcap] partial sums of squares per 16-row tile
  float* ssmlp;         // [L][d/16][bcap]
  float* qkv;           // [L][bcap][nqkv]
  float* attn_out;      // [L][bcap][qdim] attention output: GEMV input of O
  float* act;           // [L][bcap][I]    silu(gate) * up: GEMV input of down
  float* part;          // split-K partial blocks, [L + 1 (LM head)][part_blocks][1024 floats]
  float* apart;         // attention partials [L][ncu + bcap*nkv][group slots][hd + 4]
  uint32_t* banks;      // 2 banks of kShards * ctr_stride words, then keys
  uint32_t* status;     // [0] status bits, [1] abort flag
  const float* rope;    // [max_seq][hd/2][2] (cos, sin)
  const uint16_t* zero; // >= 16 zero bytes: the source of masked direct-to-LDS lanes
  // schedule
  const Task* tasks;
  const int32_t* task_off;  // [ncu + 1]
  const int32_t* expect;    // [n_counters][kShards]
  const int32_t* attn_map;  // per layer [ncu + 1]: attention slot of each CU, then the slot cap (0: none)
  int32_t ctr_stride;
  int32_t bank_words;       // words per bank (counters + keys)
  int32_t part_blocks;      // split-K partial blocks per layer
  int32_t ncu;
  int32_t nslot;
  int32_t xb_bytes;
  int32_t mfma;
  uint64_t timeout_ticks;   // s_memrealtime ticks (100 MHz)
  uint64_t* trace;          // optional per-task timestamps [ncu][trace_cap][4], NULL = off
  int32_t trace_cap;
  int32_t attn_pad;         // attention partition: empty rows ahead of each segment (upper bound)
  int32_t attn_min_rows;    // attention partition: rows a CU takes at least
  float* dump;              // optional caller buffer [L+1][bcap][d]: residual stream, tag bit cleared (NULL = off)
  // paged KV cache: K / V pools [L][nblocks][nkv][bsize][hd]; position p of
  // sequence i lives in block btab[i * bt_stride + p / bsize] at row p % bsize
  // (btab NULL: rows [L][kv_bcap][nkv][kv_scap][hd])
  const int32_t* btab;
  int32_t bt_stride, bsize, nblocks;
};

// Host planner --------------------------------------------------------------
struct PlanCfg {
  int L, d, nq, nkv, hd, I, V;
  int ncu;
  int xb_bytes;         // LDS bytes available to stage a GEMV input slice
  int mfma_min_batch;   // batch at or above which projections use MFMA tiles
  int gemv_mode = 0;    // 0: cheaper of row-owner / stream-K per stage, 1: row-owner, 2: stream-K
  double window_chunks = 6.0;  // planner cost of staging one LDS input window, in streamed chunks
  double split_chunks = 6.0;   // planner cost of splitting a stream-K group over CUs, in streamed chunks
  int ksplit_aligned = 1;      // K-split units dealt piece-aligned (each CU one input window)
  int stage_mode[6] = {0, 0, 0, 0, 0, 0};  // per stage, overrides gemv_mode when non-zero; 3: stream-K, one-tile groups
  int attn_idle = 1;    // attention prefers the CUs its layer's QKV stage left idle
  int ksplit = 1;       // K-split stages whose tasks would need many LDS input windows
  int ksplit_min_windows = 4;  // ... at least this many (per task of the tiling it replaces)
  int skip_prev = 2;    // row-owner stages skip the CUs of a previous stage that left CUs idle
                        // when the tiles per CU grow by at most skip_prev - 1 (0: never)
};
constexpr int kTaskSignal = 1;
constexpr int kTaskPublish = 2;

struct Plan {
  int batch = 0;
  int mfma = 0;
  int n_tasks = 0;
  int max_tasks_per_cu = 0;
  int n_counters = 0;
  int part_blocks = 0;                 // split-K partial blocks needed
  int grp_counters = 0;
  int grp_off[6] = {0, 0, 0, 0, 0, 0};
  int stage_tasks[6] = {0, 0, 0, 0, 0, 0};
  int stage_ksplit[6] = {0, 0, 0, 0, 0, 0};
  int stage_rows[6] = {0, 0, 0, 0, 0, 0};
  int stage_owner[6] = {0, 0, 0, 0, 0, 0};  // 1: whole sub-tiles per CU over full K (no split)
  int stage_kpieces[6] = {0, 0, 0, 0, 0, 0};  // K-split stages: K pieces (one LDS window each), else 0
  long long weight_bytes = 0;
  long long max_cu_weight_bytes = 0;
  double balance_min = 1.0;
  // flattened streams
  Task* tasks = nullptr;     // host copy, n_tasks
  int* task_off = nullptr;   // ncu + 1
  int* expect = nullptr;     // n_counters * kShards
  int* attn_map = nullptr;   // L * (ncu + 1): attention slot per CU, then the slot cap
};

// Builds and validates the per-CU streams; returns 0 or an MK_ERR_* code.
int build_plan(const PlanCfg& pc, int batch, Plan* out);
void free_plan(Plan* p);

}  // namespace mk
