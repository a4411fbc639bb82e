/* mk.h -- C ABI of an MI355X (gfx950) decode-step megakernel.
 *
 * One call of mk_decode_step runs one auto-regressive decode step of a
 * Llama/Qwen3-style decoder for a ragged batch as ONE persistent HIP launch:
 * embedding gather, per-layer RMSNorm, QKV projection, optional per-head QK
 * RMSNorm, rotate-half RoPE at each sequence's own position, KV-cache store,
 * attention over the cached positions, O projection, SwiGLU MLP, final
 * RMSNorm, LM head and greedy argmax.  This is the decode step of the
 * ForgeMegakernel paper summary ("2.1 The decode step"), kept inside one host
 * launch as its "2.3 Megakernels" section describes, with per-CU instruction
 * streams and fine-grained dependencies in place of grid-wide barriers ("4.1
 * The universal knowledge base and the milestones"; Cohere engine digest:
 * persistent kernel with one block per SM, task descriptors, counter-based
 * barriers in global memory, weights streamed before their activation
 * dependencies are met).  The dependencies are carried by the data itself:
 * every activation word handed between compute units holds a per-sequence
 * step tag in its lowest mantissa bit that the consumer polls for (see
 * mk_copy_hidden and mk_reset).
 *
 * Conventions for every entry point:
 *   - returns MK_OK (0) or a negative MK_ERR_* code; nothing aborts and no
 *     exception crosses the ABI;  mk_error_string() names a code;
 *   - "device pointer" means memory of the GPU the handle was created on;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *   - a handle may be used by one host thread / one stream at a time.
 */
#ifndef MK_H_
#define MK_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1)   /* a NULL pointer, a size out of range, batch > max_batch ... */
#define MK_ERR_UNSUPPORTED (-2)   /* a shape this build does not handle (head_dim not 64/128 ...) */
#define MK_ERR_OOM (-3)           /* device allocation failed */
#define MK_ERR_HIP (-4)           /* a HIP runtime call failed */
#define MK_ERR_PLAN (-5)          /* the schedule failed validation (never expected) */
#define MK_ERR_TOO_LARGE (-6)     /* mk_decode_step_static: the handle's scratch exceeds the static array */

/* Device status bits (mk_get_status).  Each bad value is clamped on the
 * device so nothing is read or written out of bounds. */
#define MK_STATUS_BAD_TOKEN 1u     /* tokens[i] outside [0, vocab)                  */
#define MK_STATUS_BAD_POSITION 2u  /* positions[i] outside [0, min(max_seq, seq_cap)) */
#define MK_STATUS_BAD_SEQLEN 4u    /* seq_lens[i] != positions[i] + 1               */
#define MK_STATUS_BAD_BLOCK 16u    /* mk_decode_step_paged: a block-table entry outside
                                      [0, n_blocks) (clamped) */
#define MK_STATUS_TIMEOUT 8u       /* a dependency wait exceeded the spin limit; the
                                      step was abandoned, later steps give up their waits
                                      too, and this bit stays reported until mk_reset */

typedef struct mk_handle mk_handle;   /* opaque, owned by the library */

/* Model shape.  Runtime values, not compile-time constants. */
typedef struct {
  int32_t n_layers;        /* >= 1 */
  int32_t hidden;          /* d, multiple of 64 */
  int32_t n_q_heads;       /* multiple of n_kv_heads, n_q_heads / n_kv_heads <= 8 */
  int32_t n_kv_heads;
  int32_t head_dim;        /* 64 or 128 */
  int32_t intermediate;    /* SwiGLU width, multiple of 64 */
  int32_t vocab;
  int32_t tied_embeddings; /* 1: the LM head is the embedding table */
  int32_t qk_norm;         /* 1: per-head RMSNorm of q and k before RoPE (Qwen3) */
  double rope_theta;       /* RoPE base; frequency j = theta^(-2j/head_dim), rotate-half pairs */
  float rms_eps;           /* RMSNorm epsilon (all norms) */
  int32_t max_batch;       /* 1..16: largest batch any step will use */
  int32_t max_seq;         /* positions must be < max_seq (sizes the RoPE table) */
} mk_model_cfg;

/* Weight pointers: DEVICE pointers to bf16 tensors in Hugging Face layout
 * (linear weights [out, in] row-major; norm weights [n]).  The per-layer
 * fields are HOST arrays of n_layers device pointers.  The caller owns all
 * weights; they are never copied and must outlive the handle. */
typedef struct {
  const void* embed;       /* [vocab, hidden] */
  const void* lm_head;     /* [vocab, hidden]; NULL iff tied_embeddings */
  const void* final_norm;  /* [hidden] */
  const void* const* attn_norm;  /* [hidden] */
  const void* const* q_proj;     /* [n_q_heads*head_dim, hidden] */
  const void* const* k_proj;     /* [n_kv_heads*head_dim, hidden] */
  const void* const* v_proj;     /* [n_kv_heads*head_dim, hidden] */
  const void* const* o_proj;     /* [hidden, n_q_heads*head_dim] */
  const void* const* q_norm;     /* [head_dim]; NULL array unless qk_norm */
  const void* const* k_norm;     /* [head_dim]; NULL array unless qk_norm */
  const void* const* mlp_norm;   /* [hidden] */
  const void* const* gate_proj;  /* [intermediate, hidden] */
  const void* const* up_proj;    /* [intermediate, hidden] */
  const void* const* down_proj;  /* [hidden, intermediate] */
} mk_weight_ptrs;

/* Caller-owned bf16 KV cache, DEVICE memory, layout
 * [n_layers][batch_cap][n_kv_heads][seq_cap][head_dim]; row i holds sequence
 * i.  K rows are stored after QK-norm and RoPE, V rows as projected. */
typedef struct {
  void* k;
  void* v;
  int32_t batch_cap;
  int32_t seq_cap;
} mk_kv_cache;

/* Create a handle.  The model dimensions are runtime values, so one library
 * serves every shape (the ForgeMegakernel summary, "Compiled megakernels": a
 * megakernel compiler whose constants derive from model dimensions loses
 * utilization as the model shrinks).  Validates the shape
 * (MK_ERR_UNSUPPORTED also when n_kv_heads x max_batch x max_seq reaches 2^31,
 * or when one persistent work-group does not fit a compute unit), allocates
 * the library-owned workspace (per-layer activations, partial sums, counters,
 * RoPE table) on the current HIP device, and builds, validates and uploads
 * the per-CU instruction streams of every batch size 1..max_batch (the
 * per-SM instruction streams of "4.1 The universal knowledge base and the
 * milestones"; the task descriptors of the Cohere engine digest).  It
 * synchronises the device.  *out is set only on success; on failure nothing
 * stays allocated.  Setting MK_COOP=0 in the environment switches the step
 * launches from cooperative to plain ones (then no other kernel may run on
 * the device during a step: the work-groups wait for one another). */
int mk_create(const mk_model_cfg* cfg, const mk_weight_ptrs* w, mk_handle** out);

/* One greedy decode step (the ForgeMegakernel summary, "2.1 The decode
 * step") for sequences 0..batch-1 (cache rows 0..batch-1), enqueued on
 * `stream` as ONE kernel launch ("2.3 Megakernels": the step stays within one
 * host launch); the call never allocates, copies or synchronises on the host,
 * also when the batch size differs from the previous step's (a sequence
 * joining: "3.1 Limited performance across cells", the ninth sequence).
 *   tokens[batch]     device int32: the token each sequence feeds now;
 *   positions[batch]  device int32: its decode position p_i; the new K/V row
 *                     is written to cache slot p_i and RoPE uses p_i (each
 *                     sequence its own: "3.2 Unverifiable correctness of
 *                     kernel fusing", the broadcast-position bug);
 *   seq_lens[batch]   device int32: rows attended after the write, must be
 *                     p_i + 1 (checked on the device);
 *   logits_out        device float [batch][vocab], written;
 *   next_tokens_out   device int32 [batch] greedy argmax (lowest index wins a
 *                     tie), written; may be NULL.
 * batch == 0 is a no-op.  Each call passes per-step values to its launch
 * (the sequences' step tags, the counter bank), so a launch captured into a
 * HIP graph must not be replayed as a later step.  Errors detectable on the
 * host return an error code
 * before anything is enqueued (MK_ERR_UNSUPPORTED when n_kv_heads x batch x
 * kv->seq_cap reaches 2^31: attention counts its rows in 32 bits); data
 * errors are reported by mk_get_status. */
int mk_decode_step(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                   const int32_t* seq_lens, const mk_kv_cache* kv, float* logits_out,
                   int32_t* next_tokens_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step as mk_decode_step -- same arguments, kernel, schedules and results --
 * with all the kernel's scratch (per-layer activations, split-K and attention
 * partials, counter banks) in one file-scope device array of the library, 64
 * MiB per GPU, held until the process ends, instead of the handle's
 * workspace.  It calls no allocating routine: it enqueues a fill kernel that
 * clears the used part of the array, then the step launch.  Returns
 * MK_ERR_TOO_LARGE when the handle's scratch (set by the model, max_batch and
 * the schedules) does not fit the array.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other handles)
 * race, and mk_copy_hidden / mk_copy_state / mk_copy_trace do not see a
 * static step's mid-states (mk_set_midstate_dump does).  Status bits go to
 * the handle, as for mk_decode_step. */
int mk_decode_step_static(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                          const int32_t* seq_lens, const mk_kv_cache* kv, float* logits_out,
                          int32_t* next_tokens_out, void* stream);

/* Paged KV cache (the Cohere engine digest, "Integration": compatible with
 * continuous batching and paged attention).  DEVICE pools, caller-owned:
 *   k, v          bf16 [n_layers][n_blocks][n_kv_heads][block_size][head_dim];
 *   block_table   int32 [batch][max_blocks_per_seq]: entry j of row i is the
 *                 pool block holding positions j*block_size .. +block_size-1
 *                 of the sequence in batch slot i (the same block index in
 *                 every layer's pool);
 *   block_size    positions per block, >= 64;
 *   n_blocks      blocks per layer pool (entries outside [0, n_blocks) are
 *                 clamped and raise MK_STATUS_BAD_BLOCK).
 * Positions must be < max_blocks_per_seq * block_size (else clamped,
 * MK_STATUS_BAD_POSITION).  Sequences join and leave between steps by
 * rewriting block-table rows: slot i of a step is whatever sequence the
 * caller puts there. */
typedef struct {
  void* k;
  void* v;
  const int32_t* block_table;
  int32_t n_blocks;
  int32_t block_size;
  int32_t max_blocks_per_seq;
} mk_paged_kv;

/* mk_decode_step over a paged KV cache: the same step, kernel and schedules,
 * with every cached K/V row and the new row addressed through the block
 * table.  Results are identical to mk_decode_step on a contiguous cache with
 * the same rows. */
int mk_decode_step_paged(mk_handle* h, int32_t batch, const int32_t* tokens, const int32_t* positions,
                         const int32_t* seq_lens, const mk_paged_kv* kv, float* logits_out,
                         int32_t* next_tokens_out, void* stream);

/* Copy the residual stream of the last step, enqueued on `stream` (the
 * per-layer hidden states the mid-state oracle checks: the ForgeMegakernel
 * summary, "4.2 The mid-state test oracle"):
 * dst [n_layers+1][batch][hidden] float, entry l = input of layer l (entry 0
 * is the gathered embedding, entry n_layers leaves the last layer).  The
 * kernel hands activations between compute units with a step tag in each
 * fp32 word's least significant mantissa bit; copies come back with that bit
 * cleared, the value every consumer inside the step used (so the gathered
 * bf16 embedding rows come back exactly). */
int mk_copy_hidden(mk_handle* h, int32_t batch, float* dst, void* stream);

/* Copy one per-layer mid-state buffer of the last step ("4.2 The mid-state
 * test oracle": intermediate states against float64 references), enqueued on
 * `stream`, for sequences 0..batch-1 of every layer, into dst (layout
 * [layers][batch][width], dtype as listed; tag bit cleared as above):
 *   MK_STATE_HIDDEN   float, L+1 layers, width hidden (same as mk_copy_hidden)
 *   MK_STATE_HMID     float, L, hidden: residual after attention + O proj
 *   MK_STATE_QKV      float, L, (n_q+2 n_kv) head_dim: raw q|k|v projections
 *   MK_STATE_ATTN     fp32,  L, n_q head_dim: attention output per head
 *   MK_STATE_ACT      fp32,  L, intermediate: silu(gate) * up
 * Returns MK_ERR_INVALID_ARG for an unknown `which`. */
#define MK_STATE_HIDDEN 0
#define MK_STATE_HMID 1
#define MK_STATE_QKV 2
#define MK_STATE_ATTN 3
#define MK_STATE_ACT 4
int mk_copy_state(mk_handle* h, int32_t which, int32_t batch, void* dst, void* stream);

/* In-kernel trace: where each compute unit waits (the ForgeMegakernel
 * summary, "5.2 Kernel experiment", its per-token breakdown: a megakernel's
 * synchronisation waits sit at its dependency points).  Enabled when the environment variable MK_TRACE=<n> is set
 * at mk_create; otherwise *cap = 0 and nothing is copied).  Copies, enqueued
 * on `stream`, the trace of the last step into dst (device memory of at
 * least (n_cu*cap*4 + n_cu*80)*8 bytes): for each CU and each of its first
 * `cap` tasks, 4 uint64 words {task index << 32 | layer << 16 | type << 8 | stage,
 * begin, begin again (a task polls its inputs inside its own phases), end}
 * in s_memrealtime ticks (100 MHz); then
 * 80 uint64 per CU: [0..2] ticks the loader waves waited for a free LDS
 * slot, [4..7] the compute waves waited for a loaded chunk, [8..11] the
 * compute waves waited in barriers, [12] compute wave 0's total time, [13]
 * loader wave 0's total time, [16..19] compute chunk math, [20..23] GEMV
 * input staging, [24..27] reductions and epilogues; attention phases of
 * compute wave 0 summed over layers: [32] query load and RoPE, [33] cached
 * rows, [34] merge of the waves, [35] partial publish, [36] merge of a
 * segment's partials, [37] output store, [38] completion signal, [39]
 * pieces, [40] segments finished, [41] waits for cached rows; GEMV phases of
 * compute wave 0 summed over layers, at [42 + 4 s + k] for stage s (QKV 0,
 * LM head 1, O 2, gate/up 3, down 4) and k = 0 input staging, 1 streamed
 * chunks, 2 reductions and epilogue, 3 completion signal; analysis builds
 * only: attention query preparation at [64..67] (piece setup, loads and RoPE,
 * LDS / cache stores, barrier) and QKV input staging at [68..71] (barrier,
 * loads and split, RMS scales, barrier). */
int mk_copy_trace(mk_handle* h, void* dst, int64_t bytes, int32_t* n_cu, int32_t* cap, void* stream);

/* Synchronise `stream`, return the device status bits accumulated since the
 * last call in *status and clear them, except MK_STATUS_TIMEOUT, which stays
 * set until mk_reset.  The checks behind the bits are the kernel's own input
 * validation (tokens, positions, lengths) and its bounded waits (the static
 * deadlock-freedom of the AutoMegaKernel page's schedule validator is checked
 * on the host when the schedules are built; the bound makes a wait that never
 * ends a reported error instead of a hang). */
int mk_get_status(mk_handle* h, void* stream, uint32_t* status);

/* Synchronise `stream` and clear all counters, status and the step tags of
 * the library-owned activations (needed after a MK_STATUS_TIMEOUT).  The
 * decode state itself (KV cache, positions) is the caller's, so resuming is
 * calling mk_decode_step again with the same buffers. */
int mk_reset(mk_handle* h, void* stream);

/* Context routing (the ForgeMegakernel summary, "5.3 Serving experiment" and
 * its Figure 5: kernels carry a batch size and a context bound, and requests
 * are routed among them by context length).  Declares that every later step
 * has seq_lens[i] <= max_seq_len (0 = no bound, the default): the step then
 * runs the attention partition tuned for its (batch class, context bucket)
 * -- buckets up to 128, 512, 2048 positions and beyond, batch classes below 8
 * and from 8.  The schedules and results do not depend on the bound (a
 * longer sequence is still correct, only the partition may be a poorer fit). */
int mk_set_context_bound(mk_handle* h, int32_t max_seq_len);

/* Mid-state dump: while set, every step also writes its residual stream
 * (the values mk_copy_hidden returns) into hidden_out, a DEVICE buffer the
 * caller owns, layout [n_layers+1][max_batch][hidden] float (entry l = input
 * of layer l, sequence n at row n).  The stores are the kernel's own
 * residual-stream stores with a second base pointer, inside the same launch
 * ("4.2 The mid-state test oracle": intermediate states read against float64
 * references).  NULL switches it off.  The buffer must stay valid for every
 * step enqueued while it is set. */
int mk_set_midstate_dump(mk_handle* h, float* hidden_out);

/* Free library-owned memory (workspace, schedules, trace).  The caller's
 * weights and caches are untouched. */
int mk_destroy(mk_handle* h);

/* Name of an MK_* return code (static string). */
const char* mk_error_string(int code);

/* Schedule inspection, host only (no GPU needed): build and validate the
 * per-CU instruction streams for `batch` on `n_cu` compute units (the same
 * builder mk_create uses) and report their shape and byte balance (the Cohere
 * engine digest: wave quantisation and backfilling idle SMs). */
typedef struct {
  int32_t n_tasks;
  int32_t max_tasks_per_cu;
  int32_t n_counters;
  int32_t mfma;                 /* 1 if the projection tiles use MFMA */
  int64_t weight_bytes;         /* weight bytes covered by GEMV tasks (all layers + LM head) */
  int64_t max_cu_weight_bytes;  /* largest per-CU share */
  double stage_balance_min;     /* min over GEMV stages of mean/max bytes per CU */
  int32_t stage_tasks[6];       /* tasks per layer-0 stage: QKV, ATTN, O, GU, DOWN, and LM */
  int32_t stage_ksplit[6];      /* K-splits chosen per stage (ATTN entry 0) */
  int32_t stage_rows_per_task[6];
  /* placement of layer 1 (layer 0 when there is one layer), same stage order:
   * CUs that run a task of the stage (attention: the CUs of its slot cap,
   * all CUs without a cap), and how many of them also ran the stage before
   * (QKV: the previous layer's down projection; LM head: the last one) */
  int32_t stage_cus[6];
  int32_t stage_shared_prev[6];
  int32_t attn_slot_cap;        /* attention slot cap of that layer (0: none) */
  int32_t attn_slots_valid;     /* 1: every layer's attention slots are a permutation of the CUs */
  int32_t stage_kpieces[6];     /* K-split stages: K pieces (each piece publishes partial tiles that
                                   per-CU finish tasks sum); 0 for other tilings */
} mk_plan_stats;

int mk_plan(const mk_model_cfg* cfg, int32_t batch, int32_t n_cu, mk_plan_stats* out);

/* One instruction of a CU's stream, as the kernel reads it. */
typedef struct {
  int32_t type;       /* 1 embedding gather, 2 GEMV tile, 3 attention, 4 K-split finish */
  int32_t stage;      /* 0 QKV, 1 attention, 2 O, 3 gate/up, 4 down, 5 LM head, 6 embedding */
  int32_t layer;
  int32_t row0;       /* GEMV / finish: first output row of the stage; embedding: first column */
  int32_t nsub;       /* GEMV / finish: 16-row sub-tiles; embedding: columns */
  int32_t k0, k1;     /* GEMV: K range */
  int32_t ks, nks;    /* GEMV: piece index and pieces of a split K range */
  int32_t group;      /* stream-K GEMV: row group */
  int32_t part_slot;  /* split K: first partial slot of the group (stream-K, 1024 floats) or of the
                         stage (K-split, 256-float tiles: sub-tile u's piece k at part_slot + u*nks + k) */
  int32_t nchunks;    /* weight chunks the CU's loader streams for the task */
  int32_t flags;      /* 1: the CU's last LM-head task (counts for the greedy tokens);
                         2: K-split piece (publishes partial tiles) */
} mk_task_info;

/* Schedule export, host only: the per-CU instruction streams mk_create builds
 * for `batch` on `n_cu` compute units, for inspection and for interpreting
 * the schedule on the CPU (the AutoMegaKernel page's validator proves a
 * schedule deadlock-free and race-free before it runs).  Writes the tasks of
 * CU c at tasks[cu_offsets[c] .. cu_offsets[c+1]) (cu_offsets has n_cu + 1
 * entries) and, when attn_map is not NULL, each layer's attention slots
 * [n_layers][n_cu + 1] (slot of every CU, then the slot cap, 0 = none).
 * *n_tasks receives the task count; MK_ERR_INVALID_ARG when it exceeds
 * `cap` (nothing else written). */
int mk_plan_streams(const mk_model_cfg* cfg, int32_t batch, int32_t n_cu, mk_task_info* tasks, int32_t cap,
                    int32_t* cu_offsets, int32_t* attn_map, int32_t* n_tasks);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */
