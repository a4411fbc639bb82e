// Persistent decode-step megakernel for gfx950 (MI355X).
//
// One work-group per CU walks that CU's instruction stream (built on the host,
// see mk_plan.cpp).  Inside a work-group:
//   * 3 loader waves stream every input-independent byte the CU's tasks need
//     (weight tiles, cached K/V rows) from HBM into an LDS ring with
//     non-temporal loads.  They never wait on a dependency, so weights for
//     later tasks arrive while the CU is still waiting for activations (the
//     weight prefetch of the Cohere megakernel digest; the shared-memory
//     buffer pool of the ForgeMegakernel milestones).
//   * 4 compute waves poll their step-tagged inputs until every word carries
//     this step's tag, stage the activation slice into LDS, run the GEMV
//     (VALU dot2 for small batches, MFMA 16x16x32 bf16 for batch >= 8) or
//     split-KV attention tiles out of the ring, and write their outputs with
//     fused epilogues (residual add, next RMSNorm's sum of squares, SiLU-gate,
//     RoPE, KV store, argmax).
// Cross-CU exchange uses device-coherent (sc1) loads and stores; 64-way
// sharded counters remain only for the LM head's completion (greedy tokens).
// No agent-scope cache fences are issued on the hot path.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

#include <mutex>
#include <utility>

// Per-phase timers of the in-kernel trace (per-CU stats words 32..61).  They
// cost registers in the task functions, so they are compiled only into
// analysis builds (-DMK_PHASE_TRACE=1); the per-task timestamps and the
// wait totals are always available.

namespace mk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr unsigned kCpSc1 = 16;  // cache policy: device scope (coherent across XCDs)
constexpr unsigned kCpNt = 2;    // cache policy: non-temporal (streamed once)

// Kernel arguments are read in place from the kernarg segment through a
// constant-address-space pointer; `uni` re-establishes at a function's entry
// that the pointer is wave-uniform, so every field read is a scalar load and
// never waits behind (or drains) the vector memory queue.
#define MK_AS4 __attribute__((address_space(4)))
typedef const MK_AS4 DevArgs* DArgs;
__device__ __forceinline__ DArgs uni(DArgs p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v), hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (DArgs)(((unsigned long long)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ const MK_AS4 T* as_const(const T* p) {
  return (const MK_AS4 T*)p;
}
typedef const MK_AS4 Task* TaskP;
// copy a 64-byte task descriptor out of constant memory (scalar loads)
__device__ __forceinline__ Task load_task(TaskP p) {
  // field by field (no type punning), so the copy stays in scalar registers
#define MK_TF(f) t.f = __builtin_amdgcn_readfirstlane(p->f)
  Task t;
  MK_TF(type);
  MK_TF(stage);
  MK_TF(layer);
  MK_TF(row0);
  MK_TF(nsub);
  MK_TF(k0);
  MK_TF(k1);
  MK_TF(ks);
  MK_TF(nks);
  MK_TF(group);
  MK_TF(part_slot);
  MK_TF(wait_ctr);
  MK_TF(signal_ctr);
  MK_TF(nchunks);
  MK_TF(flags);
  t.pad = 0;
#undef MK_TF
  return t;
}
__device__ __forceinline__ TaskP uni(TaskP p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v), hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (TaskP)(((unsigned long long)hi << 32) | lo);
}
constexpr uint32_t kStatusTimeout = 8u;
constexpr uint32_t kStatusBadBlock = 16u;

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7FFFFFFF, 0x00020000);
}
// device-coherent accesses; byte offsets relative to a wave-uniform base
__device__ __forceinline__ u32x4 co_load16(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ u32x2 co_load8(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ uint32_t co_load4(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ void co_store16(void* base, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ void co_store8(void* base, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ void co_store4(void* base, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rsrc(base), off, 0, kCpSc1);
}
__device__ __forceinline__ float co_loadf(const void* base, uint32_t off) { return __uint_as_float(co_load4(base, off)); }
__device__ __forceinline__ void co_storef(void* base, uint32_t off, float v) { co_store4(base, off, __float_as_uint(v)); }

// ---- step tags.  Every fp32 word one stage hands to another (residual
// stream, normalised inputs, sums of squares, q/k/v, attention outputs,
// SiLU·up) carries in its least significant mantissa bit the step tag of its
// sequence, which the host flips each step the sequence takes part in.  Each
// 4-byte word is written once per step and read whole, so a consumer polls
// the data itself until every word it needs carries this step's tag: no
// store-completion wait and no counter on a hand-off.  Consumers clear the
// bit before use (the value they see is the stored one truncated by at most
// one ulp, whatever the tag), so results do not depend on the step's tag.
__device__ __forceinline__ uint32_t tagged(float v, uint32_t tag) { return (__float_as_uint(v) & ~1u) | tag; }
__device__ __forceinline__ bool tag_ok(uint32_t w, uint32_t tag) { return (w & 1u) == tag; }
__device__ __forceinline__ bool tag_ok4(u32x4 v, uint32_t tag) {
  const uint32_t all1 = v.x & v.y & v.z & v.w, any1 = v.x | v.y | v.z | v.w;
  return ((tag ? all1 : any1) & 1u) == tag;
}
__device__ __forceinline__ void co_store_tag(void* base, uint32_t off, float v, uint32_t tag) {
  co_store4(base, off, tagged(v, tag));
}
// Consumers use a tagged word with the bit cleared, so what they compute
// does not depend on the step's tag value.
__device__ __forceinline__ uint32_t untag(uint32_t w) { return w & ~1u; }
__device__ __forceinline__ float untagf(float v) { return __uint_as_float(__float_as_uint(v) & ~1u); }
__device__ __forceinline__ u32x4 untag4(u32x4 v) { return u32x4{v.x & ~1u, v.y & ~1u, v.z & ~1u, v.w & ~1u}; }

__device__ __forceinline__ u32x4 nt_load16(const uint16_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// Bit-cast whole vectors only: clang miscompiles __builtin_bit_cast applied to
// a single ext_vector component (it reads component 0 instead).
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 x, float acc) {
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w), b = __builtin_bit_cast(bf16x8_t, x);
  acc = __builtin_amdgcn_fdot2_f32_bf16(a.s01, b.s01, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(a.s23, b.s23, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(a.s45, b.s45, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(a.s67, b.s67, acc, false);
  return acc;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

// Split 8 fp32 values into bf16 pairs hi + lo: hi is x truncated to bf16
// (exact), lo the bf16 rounding of the exact remainder x - hi, so hi + lo
// carries x to a relative 2^-17.  Two bf16 dot products (or MFMAs) then
// multiply a bf16 weight by an almost-fp32 activation.
__device__ __forceinline__ void split8(u32x4 a, u32x4 b, u32x4& hi, u32x4& lo) {
  const uint32_t x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x0 = x[2 * i], x1 = x[2 * i + 1];
    const uint32_t h0 = x0 & 0xFFFF0000u, h1 = x1 & 0xFFFF0000u;
    h[i] = (h0 >> 16) | h1;
    r[i] = f2bf(__uint_as_float(x0) - __uint_as_float(h0)) | (f2bf(__uint_as_float(x1) - __uint_as_float(h1)) << 16);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{r[0], r[1], r[2], r[3]};
}

// LDS accessors
__device__ __forceinline__ u32x4 lds_ld16(const char* p) { return *(const u32x4*)p; }
// gfx950 transposing LDS read (ds_read_b64_tr_b16): every lane loads 4
// 16-bit elements at its address; within each block of 16 lanes, lane 4a + c
// receives element c of the loads of lanes a, a + 4, a + 8 and a + 12, in that
// order (the 4 x 4 element transpose of a lane quad's 64-bit loads)
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_ld8_tr16(const char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(char*)p);
  return __builtin_bit_cast(u32x2, r);
}
__device__ __forceinline__ void lds_st16(char* p, u32x4 v) { *(u32x4*)p = v; }

// ------------------------------------------------------------ CU control
struct CState {
  uint64_t t_stream;  // trace: when the task's last chunk was consumed
  uint64_t w_empty;   // trace: ticks spent waiting for the loader
  uint64_t w_bar;     // trace: ticks spent in compute barriers
  uint64_t t_math;    // trace: ticks spent on chunk math
  uint64_t t_stage;   // trace: ticks spent staging GEMV inputs
  uint64_t t_epi;     // trace: ticks spent in reductions and epilogues
  int gen;      // compute-barrier generation
  int q;        // chunk sequence number of the current task's first chunk
  int last_dep; // unused: keeps the measured layout of the control block
  int x_stage, x_layer, x_k0, x_k1;  // signature of the staged input slice
  int synced;   // every compute wave passed a barrier after its last read of the staging buffer
  int r_stage, r_layer;              // stage whose RMS scales are in Ctrl::rms
};

struct Ctrl {
  CState cs[kComputeWaves];  // per compute wave
  int ready[kMaxSlots];
  int freed[kMaxSlots];
  int dep;  // unused (layout)
  int bar;
  int fin;  // unused (layout)
  int abort;
  unsigned long long lmkey[kMaxBatch];  // this CU's best LM-head key per sequence
  int pos[kMaxBatch];
  int slen[kMaxBatch];
  int tok[kMaxBatch];
  float rms[kMaxBatch];
#if MK_PHASE_TRACE
  uint64_t pstat[48];  // phase timers of compute wave 0, flushed at the end
  uint64_t ppack;      // the current task's phase offsets (analysis trace word 2)
  uint32_t npoll;      // polls of the current task's inputs (compute wave 0)
#endif
};

static_assert(sizeof(Ctrl) <= kCtrlBytes, "control block exceeds its LDS budget");

// Dynamic LDS of the step kernel: weight/KV ring, staged GEMV input,
// reduction scratch, control block.  Every role derives its pointers from
// this array so that LDS accesses compile to ds_* instructions.
extern __shared__ __attribute__((aligned(16))) char mk_lds[];
__device__ __forceinline__ char* xb_stage(DArgs A) { return mk_lds + (size_t)A->nslot * kSlotBytes; }
__device__ __forceinline__ float* red_scratch(DArgs A) { return (float*)(xb_stage(A) + A->xb_bytes); }
__device__ __forceinline__ Ctrl* ctrl_block(DArgs A) { return (Ctrl*)((char*)red_scratch(A) + kRedBytes); }

// Flags that order LDS accesses between the waves of one CU.  They use LDS
// instructions with an LDS-only wait (lgkmcnt): an acquire or release atomic
// at workgroup scope would also wait for every global load and store the wave
// has in flight (gfx9 counts both in vmcnt), which puts the completion of
// epilogue stores on the path of every barrier.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// read a flag; LDS reads issued after it see what was written before it was set
__device__ __forceinline__ int lds_ld_acq(int* p) {
  int v;
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
// set a flag once this wave's earlier LDS accesses are complete
__device__ __forceinline__ void lds_st_rel(int* p, int v) {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_rel(int* p, int v) {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\tds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ bool lds_aborted(Ctrl* c) { return __hip_atomic_load(&c->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0; }

__device__ __forceinline__ bool global_aborted(DArgs A) {
  return __hip_atomic_load(A->status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Every spin loop is bounded: on abort or after the time limit the CU gives
// up (the time limit also raises MK_STATUS_TIMEOUT), so the kernel always
// terminates.
struct Spin {
  uint64_t t0;
  int it;
};
__device__ __forceinline__ Spin spin_start() { return Spin{now_ticks(), 0}; }
__device__ __noinline__ bool spin_fail(const uint32_t* status, Ctrl* c) {
  if (__hip_atomic_load(&c->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return true;
  if (__hip_atomic_load(status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
    __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
  }
  return false;
}
// returns false when the wait must be abandoned
__device__ __forceinline__ bool spin_ok(DArgs A, Ctrl* c, Spin& sp) {
  if (lds_aborted(c)) return false;
  // a zero time limit (a host-forced timeout) gives up at the first failed poll
  if ((++sp.it & 63) == 0 || A->timeout_ticks == 0) {
    if (spin_fail(A->status, c)) return false;
    if (now_ticks() - sp.t0 > A->timeout_ticks) {
      atomicOr(A->status, kStatusTimeout);
      __hip_atomic_store(A->status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

// The same for loops that poll data words in global memory, with their own
// pause between polls.
#ifndef MK_POLL_SLEEP
#define MK_POLL_SLEEP 1
#endif
__device__ __forceinline__ bool poll_ok(DArgs A, Ctrl* c, Spin& sp) {
  if (lds_aborted(c)) return false;
  // a zero time limit (a host-forced timeout) gives up at the first failed poll
  if ((++sp.it & 63) == 0 || A->timeout_ticks == 0) {
    if (spin_fail(A->status, c)) return false;
    if (now_ticks() - sp.t0 > A->timeout_ticks) {
      atomicOr(A->status, kStatusTimeout);
      __hip_atomic_store(A->status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
  }
  __builtin_amdgcn_s_sleep(MK_POLL_SLEEP);
  return true;
}

// Phase-trace accumulation into the control block (LDS): no global memory
// operation, so the timers add no wait to the phases they time.
__device__ __forceinline__ void trace_add(uint64_t* p, uint64_t v) { *p += v; }
#if MK_PHASE_TRACE
#define MK_PSTAT(c, k) ((c)->pstat + (k))
#else
#define MK_PSTAT(c, k) ((uint64_t*)nullptr)
#endif

// f(integral_constant<int, 0>), f(..1), ... while f returns true: a loop
// over per-tile register arrays whose index must be a compile-time constant
// (a runtime index puts the array in scratch memory).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (void)(f(std::integral_constant<int, I>{}) && ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Software barrier among the compute waves (the loader waves never join).
__device__ __forceinline__ bool cbar(DArgs A, Ctrl* c, int& gen, int lane, uint64_t* wait_ticks = nullptr) {
  ++gen;
  if (lane == 0) lds_add_rel(&c->bar, 1);
  const int target = gen * kComputeWaves;
  if (lds_ld_acq(&c->bar) >= target) return true;
  Spin sp = spin_start();
  while (lds_ld_acq(&c->bar) < target)
    if (!spin_ok(A, c, sp)) return false;
  if (A->trace && wait_ticks) *wait_ticks += now_ticks() - sp.t0;
  return true;
}

__device__ __forceinline__ uint32_t* bank_ptr(DArgs A, int which) {
  return A->banks + (size_t)which * A->bank_words;
}
__device__ __forceinline__ unsigned long long* keys_ptr(DArgs A) {
  return (unsigned long long*)(bank_ptr(A, A->bank) + kShards * A->ctr_stride);
}

__device__ __forceinline__ void signal_counter(DArgs A, int ctr, int cu) {
  uint32_t* p = bank_ptr(A, A->bank) + (cu % kShards) * A->ctr_stride + ctr;
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------- stage geometry
__device__ __forceinline__ int stage_M(DArgs A, int st) {
  switch (st) {
    case ST_QKV: return A->nqkv;
    case ST_O: return A->d;
    case ST_GU: return 2 * A->I;
    case ST_DOWN: return A->d;
    default: return A->V;
  }
}
__device__ __forceinline__ int stage_K(DArgs A, int st) {
  switch (st) {
    case ST_O: return A->qdim;
    case ST_DOWN: return A->I;
    default: return A->d;
  }
}
// bf16 input activation [bcap][K] of a GEMV stage
__device__ __forceinline__ const float* stage_x(DArgs A, int st, int l) {
  switch (st) {
    case ST_QKV: return A->xattn + (size_t)l * A->bcap * A->d;
    case ST_O: return A->attn_out + (size_t)l * A->bcap * A->qdim;
    case ST_GU: return A->xmlp + (size_t)l * A->bcap * A->d;
    case ST_DOWN: return A->act + (size_t)l * A->bcap * A->I;
    default: return A->xattn + (size_t)A->L * A->bcap * A->d;  // LM head reads the final-normed input
  }
}
__device__ __forceinline__ const float* stage_ss(DArgs A, int st, int l) {
  const int nt = A->d / 16;
  switch (st) {
    case ST_QKV: return A->ssattn + (size_t)l * nt * A->bcap;
    case ST_GU: return A->ssmlp + (size_t)l * nt * A->bcap;
    case ST_LM: return A->ssattn + (size_t)A->L * nt * A->bcap;
    default: return nullptr;
  }
}
// weight row `lr` (logical row of the stage) of layer l.  Every candidate
// base pointer is read unconditionally (uniform scalar loads) and the row's
// matrix is chosen with selects, so a per-lane row never turns the pointer
// table read into a per-lane memory access.
__device__ __forceinline__ const uint16_t* row_ptr(DArgs A, int st, int l, int lr) {
  switch (st) {
    case ST_QKV: {
      const MK_AS4 LayerW* w = as_const(A->layers) + l;
      const uint16_t *q = w->q, *k = w->k, *v = w->v;
      const int qd = A->qdim, kd = A->kvdim;
      const bool in_q = lr < qd, in_k = !in_q && lr < qd + kd;
      const uint16_t* base = in_q ? q : (in_k ? k : v);
      const int r = in_q ? lr : (in_k ? lr - qd : lr - qd - kd);
      return base + (size_t)r * A->d;
    }
    case ST_O: return as_const(A->layers)[l].o + (size_t)lr * A->qdim;
    case ST_GU: {
      // logical tile t = 8 gate rows (8t..8t+7) followed by the same 8 up rows
      const MK_AS4 LayerW* w = as_const(A->layers) + l;
      const uint16_t *g = w->gate, *u = w->up;
      const int t = lr >> 4, j = lr & 15;
      return (j < 8 ? g : u) + (size_t)(8 * t + (j & 7)) * A->d;
    }
    case ST_DOWN: return as_const(A->layers)[l].down + (size_t)lr * A->I;
    default: return A->lm_head + (size_t)lr * A->d;
  }
}

// ---------------------------------------------------- attention partition
// The flattened attention work of a step is the (sequence, kv-head, position)
// rows in that order, each (sequence, kv-head) segment preceded by `pad`
// empty rows; CU c owns positions [W*c/ncu, W*(c+1)/ncu) of that order.
// Every CU derives the same partition from seq_lens, so a ragged batch is
// balanced without a host round trip and without broadcasting one
// sequence's position.
struct Piece {
  int i, g, j0, j1, sid, ncached, nch, has_new;
  long long seg_start;
};

// Register-resident copy of the per-sequence attended lengths (the loader
// waves must not read LDS through the compiler: see loader_main).
struct SeqLens {
  int v[kMaxBatch];
};
__device__ __forceinline__ long long attn_total_r(const SeqLens& sl, int b, int nkv) {
  long long W = 0;
#pragma unroll
  for (int i = 0; i < kMaxBatch; ++i)
    if (i < b) W += sl.v[i];
  return W * nkv;
}
__device__ __forceinline__ bool next_piece_r(const SeqLens& sl, int b, int nkv, int rpc, int pad, long long& pos,
                                             long long hi, Piece& P) {
  if (pos >= hi) return false;
  long long acc = 0;
  int i = 0, s = sl.v[0];
  bool found = false;
#pragma unroll
  for (int k = 0; k < kMaxBatch; ++k) {
    if (!found && k < b) {
      const long long seg = (long long)nkv * (sl.v[k] + pad);
      if (pos < acc + seg || k == b - 1) {
        i = k;
        s = sl.v[k];
        found = true;
      } else {
        acc += seg;
      }
    }
  }
  const int sv = s + pad;
  // off < nkv * sv < 2^31 (the host rejects larger caches): 32-bit division
  const uint32_t off = (uint32_t)(pos - acc);
  const int g = (int)(off / (uint32_t)sv);
  int jv = (int)(off - (uint32_t)g * (uint32_t)sv);
  if (jv < pad) {
    // padding ahead of the segment's rows: skip it
    if (hi - pos <= pad - jv) {
      pos = hi;
      return false;
    }
    pos += pad - jv;
    jv = pad;
  }
  long long take = sv - jv;
  if (hi - pos < take) take = hi - pos;
  P.i = i;
  P.g = g;
  P.j0 = jv - pad;
  P.j1 = P.j0 + (int)take;
  P.sid = i * nkv + g;
  P.seg_start = acc + (long long)g * sv + pad;
  const int p = s - 1;
  const int nc = (P.j1 < p ? P.j1 : p) - P.j0;
  P.ncached = nc > 0 ? nc : 0;
  P.has_new = P.j1 == s;
  P.nch = (P.ncached + rpc - 1) / rpc;
  pos += take;
  return true;
}

__device__ __forceinline__ long long attn_total(const Ctrl* c, int b, int nkv) {
  long long W = 0;
  for (int i = 0; i < b; ++i) W += c->slen[i];
  return W * nkv;
}
// First flattened row of CU cu's range, and the CU holding row x.  32-bit
// divisions when W * ncu fits (the common case), 64-bit otherwise.
__device__ __forceinline__ long long cu_lo(int cu, long long W, int ncu) {
  if ((unsigned long long)W * (unsigned)ncu <= 0xFFFFFFFFull) return (long long)((uint32_t)W * (uint32_t)cu / (uint32_t)ncu);
  return W * cu / ncu;
}
__device__ __forceinline__ int cu_of(long long x, long long W, int ncu) {
  if ((unsigned long long)W * (unsigned)ncu + (unsigned long long)W <= 0xFFFFFFFFull)
    return (int)(((uint32_t)(x + 1) * (uint32_t)ncu + (uint32_t)W - 1u) / (uint32_t)W) - 1;
  return (int)(((x + 1) * ncu + W - 1) / W) - 1;
}

// CUs that attention's rows are split over: every CU, except that a CU
// takes at least attn_min_rows rows, so that very short contexts are not cut
// into many tiny pieces whose partials must all be merged.
__device__ __forceinline__ int attn_ncu(long long W, int ncu, int min_rows) {
  const long long n = (W + min_rows - 1) / min_rows;
  return n < 1 ? 1 : (n > ncu ? ncu : (int)n);
}
// Attention works in CU slots: the schedule numbers first the CUs its layer's
// QKV stage left idle (they are already waiting, cached rows loaded), and the
// rows go to those alone when that keeps every CU at or under kAttnCapRows.
constexpr int kAttnCapRows = 256;
__device__ __forceinline__ int attn_slot(DArgs A, int l, int cu) {
  return as_const(A->attn_map)[(size_t)l * (A->ncu + 1) + cu];
}
__device__ __forceinline__ int attn_nacu(DArgs A, int l, long long W) {
  int n = attn_ncu(W, A->ncu, A->attn_min_rows);
  const int cap = as_const(A->attn_map)[(size_t)l * (A->ncu + 1) + A->ncu];
  if (cap > 0 && n > cap && (W + cap - 1) / cap <= kAttnCapRows) n = cap;
  return n;
}

// Empty rows ahead of every segment in the flattened order: a CU whose range
// crosses a segment start gets that many fewer rows for its second piece.
// At most half a CU's share (so no CU's range lies inside padding), and none
// when the padded order would leave 32-bit range.
__device__ __forceinline__ int attn_pad_rows(DArgs A, long long W, int nacu) {
  // W < 2^31 (the host rejects larger caches): 32-bit division
  uint32_t pad = (uint32_t)W / (uint32_t)(2 * nacu);
  if (pad > (uint32_t)A->attn_pad) pad = (uint32_t)A->attn_pad;
  if (W + (long long)A->b * A->nkv * pad >= (1LL << 31)) pad = 0;
  return (int)pad;
}
// flattened length of the step's attention work with `pad` empty rows per segment
__device__ __forceinline__ long long attn_padded(DArgs A, long long W, int pad) {
  return W + (long long)A->b * A->nkv * pad;
}

__device__ __forceinline__ bool next_piece(const Ctrl* c, int b, int nkv, int rpc, int pad, long long& pos, long long hi,
                                           Piece& P) {
  if (pos >= hi) return false;
  long long acc = 0;
  int i = 0;
  for (; i < b - 1; ++i) {
    const long long seg = (long long)nkv * (c->slen[i] + pad);
    if (pos < acc + seg) break;
    acc += seg;
  }
  const int s = c->slen[i], sv = s + pad;
  // off < nkv * sv < 2^31 (the host rejects larger caches): 32-bit division
  const uint32_t off = (uint32_t)(pos - acc);
  const int g = (int)(off / (uint32_t)sv);
  int jv = (int)(off - (uint32_t)g * (uint32_t)sv);
  if (jv < pad) {
    // padding ahead of the segment's rows: skip it
    if (hi - pos <= pad - jv) {
      pos = hi;
      return false;
    }
    pos += pad - jv;
    jv = pad;
  }
  long long take = sv - jv;
  if (hi - pos < take) take = hi - pos;
  P.i = i;
  P.g = g;
  P.j0 = jv - pad;
  P.j1 = P.j0 + (int)take;
  P.sid = i * nkv + g;
  P.seg_start = acc + (long long)g * sv + pad;
  const int p = s - 1;
  const int nc = (P.j1 < p ? P.j1 : p) - P.j0;
  P.ncached = nc > 0 ? nc : 0;
  P.has_new = P.j1 == s;
  P.nch = (P.ncached + rpc - 1) / rpc;
  pos += take;
  return true;
}

// ---- KV-cache rows.  Element offset (in head_dim units) of position p of
// sequence i, KV head g, layer l: contiguous rows per sequence, or a block of
// a paged pool looked up in the block table (an id outside the pool is
// clamped and raises MK_STATUS_BAD_BLOCK).
// The block table is read-only during a step.  UNIFORM = the arguments are
// the same on every lane: the entry is then read through the scalar cache,
// so the lookup never waits behind the loader's streaming loads.
template <bool UNIFORM>
__device__ __forceinline__ int kv_block(DArgs A, int i, int lb) {
  if constexpr (UNIFORM) {
    // the index through readfirstlane, so the entry comes from a scalar
    // load: a vector load here would make the loader wait for every DMA it
    // has in flight (one vmcnt) before the next chunk (measured: 13B b16
    // 17.9 -> 19.9 ms with one block per sequence)
    i = __builtin_amdgcn_readfirstlane(i);
    lb = __builtin_amdgcn_readfirstlane(lb);
  }
  const size_t idx = (size_t)i * A->bt_stride + lb;
  int blk = UNIFORM ? __builtin_amdgcn_readfirstlane(as_const(A->btab)[idx]) : A->btab[idx];
  if ((unsigned)blk >= (unsigned)A->nblocks) {
    atomicOr(A->status, kStatusBadBlock);
    blk = blk < 0 ? 0 : A->nblocks - 1;
  }
  return blk;
}
template <bool UNIFORM>
__device__ __forceinline__ size_t kv_row(DArgs A, int l, int i, int g, int p) {
  if (A->btab) {
    if constexpr (UNIFORM) p = __builtin_amdgcn_readfirstlane(p);
    const int lb = p / A->bsize;
    const int blk = kv_block<UNIFORM>(A, i, lb);
    return (((size_t)l * A->nblocks + blk) * A->nkv + g) * A->bsize + (p - lb * A->bsize);
  }
  return (((size_t)l * A->kv_bcap + i) * A->nkv + g) * A->kv_scap + p;
}

// ================================================================ loader
// The loader waves move weight tiles and cached K/V rows into the LDS ring
// with direct-to-LDS loads (global_load_lds_dwordx4): no data registers, up
// to two 16 KB chunks in flight per loader wave.  Their flag reads and
// writes go through inline LDS instructions with explicit waits: the
// compiler cannot tell a flag from the ring that the DMA writes, and would
// otherwise drain every outstanding load before each flag access.
__device__ __forceinline__ int lds_flag_read(const int* p) {
  int v;
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ void lds_flag_write(int* p, int v) {
  __asm__ volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// vmcnt <= 16 (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
__device__ __forceinline__ void wait_vmcnt16() { __builtin_amdgcn_s_waitcnt(0x4F70); }
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ void dma16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 2 /* nt */);
}

// Weight rows of one 16-row sub-tile: row j lives at (j < 8 ? b0 : b1) +
// (j & 7) * stride; rows >= nrows are past the matrix and read zeros.
struct RowBase {
  const uint16_t* b0;
  const uint16_t* b1;
  long long stride;
  int nrows;
};

__device__ __forceinline__ RowBase sub_rows(DArgs A, const Task& t, int sub) {
  const int r = t.row0 + 16 * sub;
  RowBase rb;
  rb.nrows = min(16, stage_M(A, t.stage) - r);
  const MK_AS4 LayerW* w = as_const(A->layers) + __builtin_amdgcn_readfirstlane(t.stage == ST_LM ? 0 : t.layer);
  switch (t.stage) {
    case ST_QKV: {
      const uint16_t *q = w->q, *k = w->k, *v = w->v;
      const int qd = A->qdim, kd = A->kvdim;
      const bool in_q = r < qd, in_k = !in_q && r < qd + kd;
      const uint16_t* base = in_q ? q : (in_k ? k : v);
      const int rr = in_q ? r : (in_k ? r - qd : r - qd - kd);
      rb.stride = A->d;
      rb.b0 = base + (size_t)rr * A->d;
      rb.b1 = rb.b0 + (size_t)8 * A->d;
      break;
    }
    case ST_O:
      rb.stride = A->qdim;
      rb.b0 = w->o + (size_t)r * A->qdim;
      rb.b1 = rb.b0 + (size_t)8 * A->qdim;
      break;
    case ST_GU: {
      // logical tile = 8 gate rows then the same 8 up rows
      const int t16 = r >> 4;
      rb.stride = A->d;
      rb.b0 = w->gate + (size_t)(8 * t16) * A->d;
      rb.b1 = w->up + (size_t)(8 * t16) * A->d;
      break;
    }
    case ST_DOWN:
      rb.stride = A->I;
      rb.b0 = w->down + (size_t)r * A->I;
      rb.b1 = rb.b0 + (size_t)8 * A->I;
      break;
    default:
      rb.stride = A->d;
      rb.b0 = A->lm_head + (size_t)r * A->d;
      rb.b1 = rb.b0 + (size_t)8 * A->d;
      break;
  }
  return rb;
}

// One GEMV chunk: 16 rows x 512 K, wave-load j = row j's 1 KB, contiguous in
// HBM and kRowPitch bytes apart in LDS (both the VALU and the MFMA tiles read
// this layout; a load that gathers 16 rows x 64 B per instruction instead
// streamed about 27% slower).
__device__ __forceinline__ void dma_gemv_chunk(DArgs A, const RowBase& rb, int kb, int k1, int lane, char* dst) {
  const int kk = kb * kKBlock + 8 * lane;
  const bool kok = kk < k1;
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const uint16_t* src = (j < 8 ? rb.b0 : rb.b1) + (size_t)(j & 7) * rb.stride + kk;
    dma16((kok && j < rb.nrows) ? (const void*)src : (const void*)A->zero, dst + j * kRowPitch);
  }
}

// One attention chunk: RPC cached K rows, then the same V rows.  With `rot`
// (one query head per KV head: the VALU attention tiles) row r's 16-byte
// groups are stored rotated by r & 7, so LDS position p of row r holds group
// (p + (r & 7)) mod (groups per row).
template <int HD, bool PAGED>
__device__ __forceinline__ void dma_attn_chunk(DArgs A, const uint16_t* k0, const uint16_t* v0, const uint16_t* k1,
                                               const uint16_t* v1, int split, int rows, int lane, char* dst, bool rot) {
  // rows [0, split) from k0 / v0, rows [split, rows) from k1 / v1 (a paged
  // chunk that crosses into the sequence's next block); contiguous caches
  // pass split = rows and keep one base per lane (per-lane address work runs
  // on the compute waves' SIMDs)
  constexpr int LPR = HD / 8, RP = 64 / LPR;
  const int pos = lane % LPR;
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int rl = (j & 7) * RP + lane / LPR;
    const int e = (rot ? ((pos + (rl & 7)) & (LPR - 1)) : pos) * 8;
    const uint16_t* src;
    if constexpr (PAGED) {
      const bool sec = rl >= split;
      src = (j < 8 ? (sec ? k1 : k0) : (sec ? v1 : v0)) + (uint32_t)((sec ? rl - split : rl) * HD + e);
    } else {
      src = (j < 8 ? k0 : v0) + (uint32_t)(rl * HD + e);
    }
    dma16(rl < rows ? (const void*)src : (const void*)A->zero, dst + j * 1024);
  }
}

// Wait until ring slot `slot` no longer holds an unconsumed chunk.
__device__ __forceinline__ bool loader_wait_free(DArgs A, Ctrl* c, int slot, int need, uint64_t& wait_ticks) {
  if (lds_flag_read(&c->freed[slot]) >= need) return true;
  const uint64_t t0 = now_ticks();
  for (int it = 0;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_flag_read(&c->freed[slot]) >= need) break;
    if (lds_flag_read(&c->abort)) return false;
    if (((it & 255) == 255 || A->timeout_ticks == 0) && now_ticks() - t0 > A->timeout_ticks) {
      atomicOr(A->status, kStatusTimeout);
      __hip_atomic_store(A->status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_flag_write(&c->abort, 1);
      return false;
    }
  }
  if (A->trace) wait_ticks += now_ticks() - t0;
  return true;
}

// Ring bookkeeping of one loader wave: chunk q goes to slot q % nslot; the
// chunk issued last is published (ready = q + 1) once its loads landed.
struct LoaderRing {
  int q;          // next chunk sequence number of this loader
  int slot;       // q % nslot
  int prev_slot;  // slot of the issued, not yet published chunk (-1 none)
  int prev_q;
  uint64_t wfull;
};

__device__ __forceinline__ bool ring_acquire(DArgs A, Ctrl* c, LoaderRing& R, int lane) {
  const int need = R.q - A->nslot + 1;
  if (lds_flag_read(&c->freed[R.slot]) < need) {
    // about to block: publish the chunk still in flight first, so that a
    // landed chunk never waits behind a free slot
    if (R.prev_slot >= 0) {
      wait_vmcnt0();
      if (lane == 0) lds_flag_write(&c->ready[R.prev_slot], R.prev_q + 1);
      R.prev_slot = -1;
    }
    if (!loader_wait_free(A, c, R.slot, need, R.wfull)) return false;
  }
  return true;
}
__device__ __forceinline__ void ring_issued(DArgs A, Ctrl* c, LoaderRing& R, int lane) {
  if (R.prev_slot >= 0) {
    wait_vmcnt16();  // the previous chunk's 16 loads have landed in LDS
    if (lane == 0) lds_flag_write(&c->ready[R.prev_slot], R.prev_q + 1);
  }
  R.prev_slot = R.slot;
  R.prev_q = R.q;
  R.q += kLoaderWaves;
  R.slot += kLoaderWaves;
  while (R.slot >= A->nslot) R.slot -= A->nslot;
}

__device__ __noinline__ void loader_main(DArgs A, int cu, int lw, int lane) {
  A = uni(A);
  cu = __builtin_amdgcn_readfirstlane(cu);  // wave-uniform: scalar loads, no vmcnt drain
  lw = __builtin_amdgcn_readfirstlane(lw);
  char* ring = mk_lds;
  Ctrl* c = ctrl_block(A);
  const TaskP T = as_const(A->tasks) + as_const(A->task_off)[cu];
  const int nt = as_const(A->task_off)[cu + 1] - as_const(A->task_off)[cu];
  const int rpc = 4096 / A->hd;
  // per-sequence lengths into registers before any load is in flight
  SeqLens sl;
#pragma unroll
  for (int i = 0; i < kMaxBatch; ++i) sl.v[i] = __builtin_amdgcn_readfirstlane(i < A->b ? c->slen[i] : 1);
  const uint64_t t_start = A->trace ? now_ticks() : 0;
  LoaderRing R{lw, lw % A->nslot, -1, 0, 0};
  int qbase = 0;
  for (int ti = 0; ti < nt; ++ti) {
    const Task t = load_task(uni(T + ti));
    if (t.type == TT_GEMV) {
      const int nch = t.nchunks;
      int local = R.q - qbase;
      if (local < nch) {
        int sub = local % t.nsub, kb = t.k0 / kKBlock + local / t.nsub;
        RowBase rb = sub_rows(A, t, sub);
        while (local < nch) {
          if (!ring_acquire(A, c, R, lane)) return;
          dma_gemv_chunk(A, rb, kb, t.k1, lane, ring + (size_t)R.slot * kSlotBytes);
          ring_issued(A, c, R, lane);
          local += kLoaderWaves;
          const int old_sub = sub;
          sub += kLoaderWaves;
          while (sub >= t.nsub) {
            sub -= t.nsub;
            ++kb;
          }
          if (sub != old_sub) rb = sub_rows(A, t, sub);
        }
      }
      qbase += nch;
    } else if (t.type == TT_ATTN) {
      const long long W0 = attn_total_r(sl, A->b, A->nkv);
      const int nacu = attn_nacu(A, t.layer, W0), slot = attn_slot(A, t.layer, cu);
      const int pad = attn_pad_rows(A, W0, nacu);
      const long long W = attn_padded(A, W0, pad);
      long long pos = slot < nacu ? cu_lo(slot, W, nacu) : W;
      const long long hi = slot < nacu ? cu_lo(slot + 1, W, nacu) : W;
      Piece P;
      int pbase = qbase;
      while (next_piece_r(sl, A->b, A->nkv, rpc, pad, pos, hi, P)) {
        for (int ch = R.q - pbase; ch < P.nch; ch += kLoaderWaves) {
          if (!ring_acquire(A, c, R, lane)) return;
          const int p0 = P.j0 + ch * rpc;
          const int rows = min(rpc, P.ncached - ch * rpc);
          char* dst = ring + (size_t)R.slot * kSlotBytes;
          const size_t r0 = kv_row<true>(A, t.layer, P.i, P.g, p0) * A->hd;
          // a paged chunk (at most 64 rows, blocks at least 64 positions)
          // spans at most two blocks, rows [0, split) in the first; one that
          // lies in a single block loads like a contiguous chunk
          const int split = A->btab ? min(rows, (__builtin_amdgcn_readfirstlane(p0) / A->bsize + 1) * A->bsize - p0) : rows;
          if (split < rows) {
            const size_t r1 = kv_row<true>(A, t.layer, P.i, P.g, p0 + split) * A->hd;
            if (A->hd == 128)
              dma_attn_chunk<128, true>(A, A->kc + r0, A->vc + r0, A->kc + r1, A->vc + r1, split, rows, lane, dst, A->G == 1);
            else
              dma_attn_chunk<64, true>(A, A->kc + r0, A->vc + r0, A->kc + r1, A->vc + r1, split, rows, lane, dst, A->G == 1);
          } else {
            if (A->hd == 128)
              dma_attn_chunk<128, false>(A, A->kc + r0, A->vc + r0, nullptr, nullptr, rows, rows, lane, dst, A->G == 1);
            else
              dma_attn_chunk<64, false>(A, A->kc + r0, A->vc + r0, nullptr, nullptr, rows, rows, lane, dst, A->G == 1);
          }
          ring_issued(A, c, R, lane);
        }
        pbase += P.nch;
      }
      qbase = pbase;
    }
  }
  if (R.prev_slot >= 0) {
    wait_vmcnt0();
    if (lane == 0) lds_flag_write(&c->ready[R.prev_slot], R.prev_q + 1);
  }
  if (A->trace && lane == 0) {
    uint64_t* st = A->trace + (size_t)A->ncu * A->trace_cap * 4 + (size_t)cu * kStatWords;
    st[lw] = R.wfull;
    if (lw == 0) st[13] = now_ticks() - t_start;
  }
}

// ================================================================ compute
__device__ __forceinline__ int attn_task_chunks(DArgs A, int cu, int l, int rpc) {
  A = uni(A);
  const Ctrl* c = ctrl_block(A);
  const long long W0 = attn_total(c, A->b, A->nkv);
  const int nacu = attn_nacu(A, l, W0), slot = attn_slot(A, l, cu);
  const int pad = attn_pad_rows(A, W0, nacu);
  const long long W = attn_padded(A, W0, pad);
  long long pos = slot < nacu ? cu_lo(slot, W, nacu) : W, hi = slot < nacu ? cu_lo(slot + 1, W, nacu) : W;
  Piece P;
  int n = 0;
  while (next_piece(c, A->b, A->nkv, rpc, pad, pos, hi, P)) n += P.nch;
  return n;
}

__device__ __forceinline__ bool wait_chunk(DArgs A, Ctrl* c, int gq, uint64_t& wait_ticks) {
  const int slot = gq % A->nslot;
  if (lds_ld_acq(&c->ready[slot]) >= gq + 1) return true;
  Spin sp = spin_start();
  while (lds_ld_acq(&c->ready[slot]) < gq + 1)
    if (!spin_ok(A, c, sp)) return false;
  if (A->trace) wait_ticks += now_ticks() - sp.t0;
  return true;
}
__device__ __forceinline__ void free_chunk(DArgs A, Ctrl* c, int gq, int lane) {
  if (lane == 0) lds_st_rel(&c->freed[gq % A->nslot], gq + 1);
}

// Wave-wide sum over 16-lane groups (lanes l, l^1, ..., l^8).
// DPP lane moves within 16-lane rows: quad_perm [1,0,3,2] (lane ^ 1),
// quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (lane i of each 8 <- 7-i),
// row_mirror (lane i of each 16 <- 15-i), row_ror:8 (lane ^ 8).
// A DPP move reads other lanes' registers, so it must run with every lane of
// the wave active.  Callers use its result unconditionally (never as one arm
// of a select: the compiler may turn that into a branch, and a move reading
// a lane switched off by the branch returns 0).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// row_ror:n moves lane (i - n) mod 16 of each row into lane i; row_shl:n
// moves lane i + n and row_shr:n lane i - n (0 past the row's ends).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140, kDppShl4 = 0x104,
              kDppShr4 = 0x114, kDppRor8 = 0x128;
// Sum over aligned groups of N lanes (N = 2, 4, 8 or 16); every lane of a
// group gets the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2..16 lanes");
  v += dpp_f<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float sum16(float v) { return group_sum<16>(v); }

// Order-preserving 64-bit key: larger logit first, then lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  v = v + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (uint32_t)idx);
}

// Lane exchanges across 16-lane rows with the VALU lane-swap instructions
// (no LDS round trip).  permlane16_swap(a, b) returns ([a r0, b r0, a r2,
// b r2], [a r1, b r1, a r3, b r3]) by 16-lane row; permlane32_swap(a, b)
// returns ([a lo, b lo], [a hi, b hi]) by 32-lane half.  So x + y of a swap of
// (a, b) is, on each lane, a + a' on the lower row (half) of a pair and
// b + b' on the upper one, where ' is the partner lane (lane ^ 16 / ^ 32).
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float a) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float a) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sequence n's per-16-row partial sums of squares (nt <= 64 * kSsLoads of
// them, entry lane + 64 k in u[k]), polled until each carries the sequence's
// step tag.  `loaded`: u already holds a first attempt.  Entries past nt hold
// the tag itself.
constexpr int kSsLoads = 8;  // hidden <= 8192
__device__ __forceinline__ bool poll_ss(DArgs A, Ctrl* c, const float* ss, int n, int nt, uint32_t tag, int lane,
                                        uint32_t (&u)[kSsLoads], bool loaded) {
  Spin sp = spin_start();
  for (;;) {
    if (!loaded) {
#pragma unroll
      for (int k = 0; k < kSsLoads; ++k) {
        const int i = lane + 64 * k;
        u[k] = i < nt ? co_load4(ss, (uint32_t)(((size_t)i * A->bcap + n) * 4)) : tag;
      }
    }
    loaded = false;
    bool ok = true;
#pragma unroll
    for (int k = 0; k < kSsLoads; ++k) ok = ok & tag_ok(u[k], tag);
    if (__all(ok)) return true;
    if (!poll_ok(A, c, sp)) return false;
  }
}

// RMS scales of sequences w, w + 4, ... (< b) into the control block: all
// their per-16-row sums of squares are loaded in one batch and polled until
// each carries its sequence's step tag (one memory round trip for up to four
// sequences per wave).  `first` holds a first attempt for sequence w when
// `loaded`.
__device__ __forceinline__ bool rms_scales(DArgs A, Ctrl* c, const float* ss, int w, int lane, uint32_t tags,
                                           const uint32_t (&first)[kSsLoads], bool loaded) {
  constexpr int kSeq = kMaxBatch / kComputeWaves;
  const int nt = A->d / 16;
  uint32_t u[kSeq][kSsLoads];
  Spin sp = spin_start();
  for (;;) {
#pragma unroll
    for (int j = 0; j < kSeq; ++j) {
      const int n = w + kComputeWaves * j;
      const uint32_t tg = (tags >> n) & 1u;
#pragma unroll
      for (int k = 0; k < kSsLoads; ++k) {
        const int i = lane + 64 * k;
        if (j == 0 && loaded) u[j][k] = first[k];
        else u[j][k] = (n < A->b && i < nt) ? co_load4(ss, (uint32_t)(((size_t)i * A->bcap + n) * 4)) : tg;
      }
    }
    loaded = false;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < kSeq; ++j) {
      const uint32_t tg = (tags >> (w + kComputeWaves * j)) & 1u;
#pragma unroll
      for (int k = 0; k < kSsLoads; ++k) ok = ok & tag_ok(u[j][k], tg);
    }
    if (__all(ok)) break;
    if (!poll_ok(A, c, sp)) return false;
  }
#pragma unroll
  for (int j = 0; j < kSeq; ++j) {
    const int n = w + kComputeWaves * j;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kSsLoads; ++k) acc += lane + 64 * k < nt ? __uint_as_float(untag(u[j][k])) : 0.f;
    acc = group_sum<16>(acc);
    acc = swap16_sum(acc, acc);
    acc = swap32_sum(acc, acc);
    if (lane == 0 && n < A->b) c->rms[n] = 1.0f / sqrtf(acc / (float)A->d + A->eps);
  }
  return true;
}

// ---- stage the GEMV input slice x[n][kk0:kk1) (bf16, n < b) into LDS with
//      rows padded to kk1-kk0+8 elements, and the RMS scales of stages that
//      normalize their input.  Skipped when the same slice is already staged.
//      The input words are polled until they carry the step tag.
#ifndef MK_STAGE_BATCH_MFMA
#define MK_STAGE_BATCH_MFMA 4
#endif
template <int kStageBatch>
__device__ __forceinline__ bool stage_input(DArgs A, const Task& t, int kk0, int kk1, char* xb, Ctrl* c, CState& s, int w,
                            int lane, bool want_rms = true) {
  if (s.x_stage == t.stage && s.x_layer == t.layer && s.x_k0 == kk0 && s.x_k1 == kk1) return true;
  // analysis builds: sub-phases of the QKV staging (compute wave 0)
  uint64_t* sp = (MK_PHASE_TRACE && A->trace && w == 0 && lane == 0 && t.stage == ST_QKV) ? MK_PSTAT(c, 36) : nullptr;
  uint64_t ts = sp ? now_ticks() : 0;
  auto smark = [&](int k) {
    if (sp) {
      const uint64_t tn = now_ticks();
      trace_add(sp + k, tn - ts);
      ts = tn;
    }
  };
  // every compute wave must be done reading the previous slice (already
  // true right after a task that ended with a barrier)
  if (!s.synced && !cbar(A, c, s.gen, lane, &s.w_bar)) return false;
  s.synced = 0;
  smark(0);
  // the fp32 input slice as bf16 hi and lo halves: [n][ksp] hi, then [n][ksp] lo
  const int K = stage_K(A, t.stage);
  const int ksl = kk1 - kk0, ksp = ksl + 8;
  const float* x = stage_x(A, t.stage, t.layer);
  char* xlo = xb + (size_t)A->b * ksp * 2;
  const int per_row = ksl / 8;
  const int units = A->b * per_row;
  const int tid = w * 64 + lane;
  const uint32_t tags = A->rowtag;
  // RMS partial sums of sequence w, first attempt in flight with the input
  const float* ss = stage_ss(A, t.stage, t.layer);
  const bool rms = want_rms && ss && !(s.r_stage == t.stage && s.r_layer == t.layer);
  const int nt = A->d / 16;
  const uint32_t tw = (tags >> w) & 1u;
  uint32_t ssu[kSsLoads];
#pragma unroll
  for (int k = 0; k < kSsLoads; ++k) {
    const int i = lane + 64 * k;
    ssu[k] = (rms && w < A->b && i < nt) ? co_load4(ss, (uint32_t)(((size_t)i * A->bcap + w) * 4)) : tw;
  }
  // up to kStageBatch units per thread in flight at once: one memory round
  // trip per batch rather than per unit; the batch is loaded again until
  // every word carries its sequence's tag
  for (int u0 = tid; u0 < units; u0 += kStageBatch * kComputeThreads) {
    u32x4 va[kStageBatch], vb[kStageBatch];
    Spin sp = spin_start();
    for (;;) {
#if MK_PHASE_TRACE
      if (A->trace && w == 0 && lane == 0) c->npoll += 1;
#endif
      bool ok = true;
#pragma unroll
      for (int k = 0; k < kStageBatch; ++k) {
        const int u = u0 + k * kComputeThreads;
        const int n = u / per_row, kq = u - n * per_row;
        const uint32_t off = (uint32_t)(((size_t)n * K + kk0 + 8 * kq) * 4);
        va[k] = vb[k] = u32x4{0, 0, 0, 0};
        if (u < units) {
          va[k] = co_load16(x, off);
          vb[k] = co_load16(x, off + 16);
        }
      }
#pragma unroll
      for (int k = 0; k < kStageBatch; ++k) {
        const int u = u0 + k * kComputeThreads;
        const uint32_t tg = (tags >> (u / per_row)) & 1u;
        if (u < units) ok = ok & tag_ok4(va[k], tg) & tag_ok4(vb[k], tg);
      }
      if (__all(ok)) break;
      if (!poll_ok(A, c, sp)) return false;
    }
#pragma unroll
    for (int k = 0; k < kStageBatch; ++k) {
      const int u = u0 + k * kComputeThreads;
      const int n = u / per_row, kq = u - n * per_row;
      if (u < units) {
        u32x4 hi, lo;
        split8(untag4(va[k]), untag4(vb[k]), hi, lo);
        lds_st16(xb + ((size_t)n * ksp + 8 * kq) * 2, hi);
        lds_st16(xlo + ((size_t)n * ksp + 8 * kq) * 2, lo);
      }
    }
  }
  smark(1);
  if (rms) {
    for (int n = w; n < A->b; n += kComputeWaves) {
      if (!poll_ss(A, c, ss, n, nt, (tags >> n) & 1u, lane, ssu, n == w)) return false;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < kSsLoads; ++k) acc += lane + 64 * k < nt ? __uint_as_float(untag(ssu[k])) : 0.f;
      acc = group_sum<16>(acc);
      acc = swap16_sum(acc, acc);
      acc = swap32_sum(acc, acc);
      if (lane == 0) c->rms[n] = 1.0f / sqrtf(acc / (float)A->d + A->eps);
    }
    s.r_stage = t.stage;
    s.r_layer = t.layer;
  }
  s.x_stage = t.stage;
  s.x_layer = t.layer;
  s.x_k0 = kk0;
  s.x_k1 = kk1;
  smark(2);
  const bool ok = cbar(A, c, s.gen, lane, &s.w_bar);
  smark(3);
  return ok;
}

// ---- VALU chunk: 16 rows x 512 K; lane l covers K elements [8l, 8l+8)
//      (input as bf16 hi + lo halves, xlo_off bytes apart in LDS)
template <int NB>
__device__ __forceinline__ void valu_chunk(const char* slot, const char* xb, int xlo_off, int ksp, int kl, int klen,
                                           int lane, float (&acc)[16][NB]) {
  u32x4 xh[NB], xl[NB];
  const bool ok = kl < klen;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    xh[n] = ok ? lds_ld16(xb + ((size_t)n * ksp + kl) * 2) : u32x4{0, 0, 0, 0};
    xl[n] = ok ? lds_ld16(xb + xlo_off + ((size_t)n * ksp + kl) * 2) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    u32x4 wv = lds_ld16(slot + j * kRowPitch + lane * 16);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[j][n] = dot8_bf16(wv, xh[n], dot8_bf16(wv, xl[n], acc[j][n]));
  }
}

// Reduce acc[16][NB] over the 64 lanes with a transposing butterfly; lane l
// ends with the total of row ((l>>5)&1)*8 + ((l>>4)&1)*4 + ((l>>3)&1)*2 + ((l>>2)&1).
template <int NB>
__device__ __forceinline__ void valu_reduce(float (&acc)[16][NB], int lane, float* out /*[NB]*/) {
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    float v8[8], v4[4], v2[2], v1;
    const bool b3 = lane & 8, b2 = lane & 4;
    // lane ^ 32: the lower half keeps rows r, the upper half rows r + 8
#pragma unroll
    for (int r = 0; r < 8; ++r) v8[r] = swap32_sum(acc[r][n], acc[r + 8][n]);
    // lane ^ 16: even rows of 16 lanes keep r, odd ones r + 4
#pragma unroll
    for (int r = 0; r < 4; ++r) v4[r] = swap16_sum(v8[r], v8[r + 4]);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float send = b3 ? v4[r] : v4[r + 2];
      float keep = b3 ? v4[r + 2] : v4[r];
      v2[r] = keep + dpp_f<kDppRor8>(send);  // lane ^ 8
    }
    {
      float send = b2 ? v2[0] : v2[1];
      float keep = b2 ? v2[1] : v2[0];
      // lane ^ 4 within a 16-lane row: lanes with bit 2 clear read lane + 4,
      // the others lane - 4.  Both moves run on every lane with the unwanted
      // direction zeroed at the source (a select between two moved values
      // may be turned into a branch, and a move that reads a lane switched
      // off by the branch returns 0).
      const float s_up = b2 ? send : 0.f, s_dn = b2 ? 0.f : send;
      v1 = keep + dpp_f<kDppShl4>(s_up) + dpp_f<kDppShr4>(s_dn);
    }
    v1 += dpp_f<kDppXor2>(v1);
    v1 += dpp_f<kDppXor1>(v1);
    out[n] = v1;
  }
}

// ---- MFMA chunk: one 16-row sub-tile x 16 k-steps of 32; B operand (the
//      input, batch padded to 16 with zeros) from the staged LDS slice.
//      The input is bf16 hi + lo halves (xlo_off bytes apart): two MFMAs per
//      k-step into the same accumulator.
__device__ __forceinline__ void mfma_chunk(const char* slot, const char* xb, int xlo_off, int ksp, int kl, int klen, int b,
                                           int lane, f32x4& acc) {
  // columns n >= b of the B operand repeat column b - 1: their outputs are
  // never stored, and every LDS read stays inside the staged rows
  const int n = min(lane & 15, b - 1), kq = 8 * (lane >> 4);
  const char* xh = xb + ((size_t)n * ksp + kl + kq) * 2;
  const char* xl = xh + xlo_off;
  // A operand of k-step s: row lane & 15, K elements 32 s + 8 (lane >> 4) .. + 7
  const char* wv = slot + (lane & 15) * kRowPitch + (lane >> 4) * 16;
  f32x4 alo = {0.f, 0.f, 0.f, 0.f};  // the lo halves accumulate separately (two independent MFMA chains)
  if (kl + kKBlock <= klen) {
    // whole 512-wide block: LDS reads four K-steps at a time ahead of their MFMAs
#pragma unroll
    for (int s0 = 0; s0 < kWaveLoads; s0 += 4) {
      u32x4 bh[4], bl[4], av[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = lds_ld16(wv + (s0 + u) * 64);
        bh[u] = lds_ld16(xh + (s0 + u) * 64);
        bl[u] = lds_ld16(xl + (s0 + u) * 64);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        alo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]), __builtin_bit_cast(bf16x8_t, bl[u]),
                                                      alo, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]), __builtin_bit_cast(bf16x8_t, bh[u]),
                                                      acc, 0, 0, 0);
      }
    }
  } else {
    // the ragged last block of K: steps of 32 up to klen (klen - kl is a multiple of 32)
    for (int s = 0; s < kWaveLoads && kl + 32 * s < klen; ++s) {
      const u32x4 av = lds_ld16(wv + s * 64), bh = lds_ld16(xh + s * 64), bl = lds_ld16(xl + s * 64);
      alo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bl), alo,
                                                    0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bh), acc,
                                                    0, 0, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] += alo[q];
}

// Where a GEMV stage's epilogue writes, computed once per task (wave-uniform
// values, so the per-element code issues no kernel-argument loads).
struct EpiCtx {
  int stage, M, b, bcap, ostride;
  uint32_t tags;  // per-sequence step tags of the stored words
  float* out;    // QKV: qkv rows; O: mid-layer residual; DOWN: next residual; GU: SiLU·up; LM: logits
  float* xo;     // O / DOWN: the next RMSNorm's input
  float* ssout;  // O / DOWN: its per-16-row sums of squares
  float* dump;   // DOWN: the caller's mid-state dump of this layer's output (NULL = none)
};
__device__ __forceinline__ EpiCtx make_epi(DArgs A, const Task& t) {
  EpiCtx e;
  const int l = t.layer;
  e.stage = t.stage;
  e.M = stage_M(A, t.stage);
  e.b = A->b;
  e.bcap = A->bcap;
  e.tags = A->rowtag;
  e.xo = e.ssout = e.dump = nullptr;
  switch (t.stage) {
    case ST_QKV:
      e.out = A->qkv + (size_t)l * A->bcap * A->nqkv;
      e.ostride = A->nqkv;
      break;
    case ST_O:
      e.out = A->hmid + (size_t)l * A->bcap * A->d;
      e.xo = A->xmlp + (size_t)l * A->bcap * A->d;
      e.ssout = A->ssmlp + (size_t)l * (A->d / 16) * A->bcap;
      e.ostride = A->d;
      break;
    case ST_DOWN:
      e.out = A->hres + (size_t)(l + 1) * A->bcap * A->d;
      e.xo = A->xattn + (size_t)(l + 1) * A->bcap * A->d;
      e.ssout = A->ssattn + (size_t)(l + 1) * (A->d / 16) * A->bcap;
      e.dump = A->dump ? A->dump + (size_t)(l + 1) * A->bcap * A->d : nullptr;
      e.ostride = A->d;
      break;
    case ST_GU:
      e.out = A->act + (size_t)l * A->bcap * A->I;
      e.ostride = A->I;
      break;
    default:
      e.out = A->logits;
      e.ostride = A->V;
      break;
  }
  return e;
}

// Epilogue of one output element (row `lr` of the stage, sequence n) of a
// complete sub-tile.  Lanes map to (row = lane & 15, n), so each 16-lane
// group holds one sequence's 16 consecutive rows.  `resid` is the residual
// prefetched for O / DOWN, `nw` the next norm's weight of row lr, `rms` the
// RMS scale of sequence n for the stages that normalise their input.
__device__ __forceinline__ void gemv_epilogue(const EpiCtx& e, Ctrl* c, int lr, int row, int n, float val, float val_up,
                                              float resid, float nw, float rms) {
  const bool valid = n < e.b && lr < e.M;
  const uint32_t off = (uint32_t)(((size_t)n * e.ostride + lr) * 4);
  const uint32_t tg = (e.tags >> n) & 1u;
  switch (e.stage) {
    case ST_QKV:
      if (valid) co_store_tag(e.out, off, rms * val, tg);
      break;
    case ST_O:
    case ST_DOWN: {
      // h = residual + projection; also the next RMSNorm's input and its
      // per-16-row sum of squares.
      float h = valid ? resid + val : 0.f;
      const float xn = valid ? h * nw : 0.f;
      if (valid) {
        co_store_tag(e.out, off, h, tg);
        co_store_tag(e.xo, off, xn, tg);
        // the mid-state dump holds the value consumers use (tag bit cleared)
        if (e.dump) e.dump[(size_t)n * e.ostride + lr] = untagf(h);
      }
      float ss = sum16(h * h);
      if (valid && row == 0) co_store_tag(e.ssout, (uint32_t)((((size_t)lr >> 4) * e.bcap + n) * 4), ss, tg);
      break;
    }
    case ST_GU: {
      // rows 0-7 of a 16-row logical tile are gate rows, 8-15 the same up rows
      if (valid && row < 8) {
        const float g = rms * val, u = rms * val_up;
        const float a = g / (1.0f + __expf(-g)) * u;
        co_store_tag(e.out, (uint32_t)(((size_t)n * e.ostride + 8 * (lr >> 4) + row) * 4), a, tg);
      }
      break;
    }
    default: {  // LM head + greedy argmax
      const float v = valid ? rms * val : 0.f;
      if (valid) e.out[(size_t)n * e.ostride + lr] = v;
      // every lane folds its key into the CU's best key of sequence n (an
      // LDS atomic max with no return: no wait, no cross-lane reduction)
      if (valid) __hip_atomic_fetch_max(&c->lmkey[n], argmax_key(v, lr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      break;
    }
  }
}

// One GEMV task: nsub 16-row sub-tiles over K range [k0, k1).  Compute wave
// w owns sub-tiles w, w+4, ... (at most tiles_per_wave(NB) of them): it
// consumes their chunks, reduces each across its own lanes and runs the
// epilogue, with no cross-wave reduction.  A sub-tile whose K range is split
// over several tasks (nks > 1, one sub-tile per wave) publishes partials; the
// last piece to finish sums them in piece order and runs the epilogue.
// NB > 0: VALU dot products for NB sequences; NB == 0: MFMA (batch <= 16).
template <int NB>
__device__ __noinline__ bool gemv_task(DArgs A, TaskP tp, int cu, int w, int lane) {
  constexpr int TPW = tiles_per_wave(NB);
  constexpr int NV = NB > 0 ? NB : 1;
  constexpr int kResidTiles = 2;  // owned sub-tiles whose residual is prefetched
  A = uni(A);
  if constexpr (NB == 0) {
    // wave-uniform: scalar loads, no vmcnt drain (the VALU instantiations run
    // slower with these in scalar registers: measured on the b1 models)
    cu = __builtin_amdgcn_readfirstlane(cu);
    w = __builtin_amdgcn_readfirstlane(w);
  }
  char* ring = mk_lds;
  char* xb = xb_stage(A);
  float* red = red_scratch(A);
  Ctrl* c = ctrl_block(A);
  CState& s = c->cs[w];
  const Task t = load_task(uni(tp));
  const int nsub = t.nsub;
  // Fewer sub-tiles than compute waves: the waves of one sub-tile split its
  // K blocks (wave w takes sub-tile w % nsub, blocks kb = w / nsub mod S) and
  // sum their partial tiles in LDS before the epilogue.
  const int S = nsub == 1 ? kComputeWaves : (nsub == 2 ? kComputeWaves / 2 : 1);
  const int kpart = S > 1 ? w / nsub : 0;
  const int msub = S > 1 ? w % nsub : w;  // this wave's (first) sub-tile
  const int nown = S > 1 ? 1 : (nsub > w ? min(TPW, (nsub - w + kComputeWaves - 1) / kComputeWaves) : 0);
  const int M = stage_M(A, t.stage);
  const int nkb = (t.k1 - t.k0 + kKBlock - 1) / kKBlock;
  const int row = lane & 15;
  // a K-split piece publishes its partial tiles; the stage's finish tasks run the epilogue
  const bool publish = (t.flags & kTaskPublish) != 0;
  const bool has_resid = !publish && (t.stage == ST_O || t.stage == ST_DOWN);
  const float* hin = t.stage == ST_DOWN ? A->hmid + (size_t)t.layer * A->bcap * A->d
                                        : A->hres + (size_t)t.layer * A->bcap * A->d;
  auto tile_row0 = [&](int i) { return t.row0 + 16 * (msub + kComputeWaves * i); };
  // residuals and next-norm weights of the first owned rows, prefetched
  // while the weights stream (only the wave that runs the epilogue needs them)
  const bool lead = kpart == 0;
  const uint16_t* nwp = nullptr;
  if (t.stage == ST_O) nwp = as_const(A->layers)[t.layer].mlp_norm;
  if (t.stage == ST_DOWN) nwp = t.layer + 1 < A->L ? as_const(A->layers)[t.layer + 1].attn_norm : A->final_norm;
  float resid[kResidTiles][4], nwv[kResidTiles];
#pragma unroll
  for (int i = 0; i < kResidTiles; ++i) {
    const int lr = tile_row0(i) + row;
    nwv[i] = (has_resid && lead && i < nown && lr < M) ? bf2f(nwp[lr]) : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      resid[i][j] = 0.f;
      const int n = (lane >> 4) + 4 * j;
      if (has_resid && lead && i < nown && n < A->b && lr < M) resid[i][j] = co_loadf(hin, (uint32_t)(((size_t)n * A->d + lr) * 4));
    }
  }
  // trace: GEMV phase totals of compute wave 0, per stage (per-CU stats words
  // 42 + 4 * stage + {0 staging, 1 chunks, 2 reduce + epilogue, 3 signal})
  uint64_t* gst = (MK_PHASE_TRACE && A->trace && w == 0 && lane == 0)
                      ? MK_PSTAT(c, 10 + 4 * (t.stage == ST_LM ? 1 : t.stage))
                      : nullptr;
  uint64_t gt = gst ? now_ticks() : 0;
  const uint64_t gt0 = gt;
  uint64_t gpack = 0;
  auto gmark = [&](int k) {
    if (gst) {
      const uint64_t tn = now_ticks();
      trace_add(gst + k, tn - gt);
      gt = tn;
      // per-task offsets of the first staging, the chunks and the epilogue
      if (k < 3 && !((gpack >> (16 * k)) & 0xFFFF)) gpack |= ((tn - gt0) & 0xFFFF) << (16 * k);
    }
  };
  float vacc[TPW][16][NV];
  f32x4 macc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    macc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int n = 0; n < NV; ++n) vacc[i][j][n] = 0.f;
  }
  // K windows that fit the LDS staging buffer
  // (4 bytes per staged element: bf16 hi + lo)
  int wkb = ((A->xb_bytes / (4 * A->b)) - 8) / kKBlock;
  if (wkb < 1) wkb = 1;
  for (int wb = 0; wb < nkb; wb += wkb) {
    const int we = min(nkb, wb + wkb);
    const int kk0 = t.k0 + wb * kKBlock, kk1 = min(t.k1, t.k0 + we * kKBlock);
    const uint64_t ts0 = A->trace ? now_ticks() : 0;
    if (!stage_input<NB == 0 ? MK_STAGE_BATCH_MFMA : 4>(A, t, kk0, kk1, xb, c, s, w, lane, !publish)) return false;
    if (A->trace) s.t_stage += now_ticks() - ts0;
    gmark(0);
    const int ksp = kk1 - kk0 + 8, klen = kk1 - kk0, xlo_off = A->b * ksp * 2;
    // first block of this window that belongs to this wave's K part
    const int kb0 = S > 1 ? wb + ((kpart - wb) % S + S) % S : wb;
    for (int kb = kb0; kb < we && nown > 0; kb += S) {
      const int kl = (kb - wb) * kKBlock;
      if constexpr (NB > 0) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          if (i >= nown) break;
          const int gq = s.q + kb * nsub + msub + kComputeWaves * i;
          if (!wait_chunk(A, c, gq, s.w_empty)) return false;
          const char* slot = ring + (size_t)(gq % A->nslot) * kSlotBytes;
          const uint64_t tm0 = A->trace ? now_ticks() : 0;
          valu_chunk<NB>(slot, xb, xlo_off, ksp, kl + 8 * lane, klen, lane, vacc[i]);
          free_chunk(A, c, gq, lane);
          if (A->trace) s.t_math += now_ticks() - tm0;
        }
      } else {
        // eight MFMA tiles per wave: a plain unrolled loop with an early exit
        // is not always unrolled, and a runtime index would move the
        // accumulators to scratch memory
        bool ok = true;
        static_for<TPW>([&](auto I) {
          constexpr int i = decltype(I)::value;
          if (i >= nown) return false;
          const int gq = s.q + kb * nsub + msub + kComputeWaves * i;
          if (!wait_chunk(A, c, gq, s.w_empty)) return ok = false;
          const char* slot = ring + (size_t)(gq % A->nslot) * kSlotBytes;
          const uint64_t tm0 = A->trace ? now_ticks() : 0;
          mfma_chunk(slot, xb, xlo_off, ksp, kl, klen, A->b, lane, macc[i]);
          free_chunk(A, c, gq, lane);
          if (A->trace) s.t_math += now_ticks() - tm0;
          return true;
        });
        if (!ok) return false;
      }
    }
  }
  const uint64_t te0 = A->trace ? now_ticks() : 0;
  gmark(1);
  // Land the prefetched residuals and norm weights now, while no store is in
  // flight: a first use after the epilogue's stores would make the wait on
  // them also wait for those stores.  Residual words without this step's tag
  // are loaded again.
#pragma unroll
  for (int i = 0; i < kResidTiles; ++i) asm volatile("" ::"v"(nwv[i]));
  if (has_resid && lead) {
    const uint32_t tags = A->rowtag;
    Spin sp = spin_start();
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < kResidTiles; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = (lane >> 4) + 4 * j;
          if (i < nown && n < A->b && tile_row0(i) + row < M)
            ok = ok & tag_ok(__float_as_uint(resid[i][j]), (tags >> n) & 1u);
        }
      if (__all(ok)) break;
      if (!poll_ok(A, c, sp)) return false;
#pragma unroll
      for (int i = 0; i < kResidTiles; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = (lane >> 4) + 4 * j, lr = tile_row0(i) + row;
          if (i < nown && n < A->b && lr < M) resid[i][j] = co_loadf(hin, (uint32_t)(((size_t)n * A->d + lr) * 4));
        }
    }
#pragma unroll
    for (int i = 0; i < kResidTiles; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) resid[i][j] = untagf(resid[i][j]);
  }
  // owned sub-tile i's totals -> this wave's LDS scratch as [16 rows][16 n],
  // read back with lanes mapped to (row = lane & 15, n = lane / 16 + 4 j)
  float* rw = red + w * 256;
  auto tile_values = [&](int i, float (&val)[4], float (&up)[4]) {
    if constexpr (NB > 0) {
      float tot[NB];
      valu_reduce<NB>(vacc[i], lane, tot);
      if ((lane & 3) == 0) {
        const int rr = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
#pragma unroll
        for (int n = 0; n < NB; ++n) rw[rr * 16 + n] = tot[n];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[(4 * (lane >> 4) + q) * 16 + (lane & 15)] = macc[i][q];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (lane >> 4) + 4 * j;
      val[j] = rw[row * 16 + n];
      up[j] = (t.stage == ST_GU && row < 8) ? rw[(row + 8) * 16 + n] : 0.f;
    }
  };
  // K split inside the CU: every wave leaves its partial tile in its LDS
  // scratch (tile_values), then the leading wave of each sub-tile adds the
  // others' in a fixed order
  float sval[4] = {0.f, 0.f, 0.f, 0.f}, sup[4] = {0.f, 0.f, 0.f, 0.f};
  // analysis builds: QKV reduction sub-phases (tile values, barrier, combine, epilogue)
  uint64_t* rsp = (MK_PHASE_TRACE && gst && t.stage == ST_QKV) ? MK_PSTAT(c, 42) : nullptr;
  uint64_t tr0 = rsp ? now_ticks() : 0;
  auto rmark = [&](int k) {
    if (rsp) {
      const uint64_t tn = now_ticks();
      trace_add(rsp + k, tn - tr0);
      tr0 = tn;
    }
  };
  if (S > 1) {
    tile_values(0, sval, sup);
    rmark(0);
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    rmark(1);
    if (lead) {
      // every partial read first (one LDS wait), then summed in wave order
      const bool gu = t.stage == ST_GU && row < 8;
      float pv[kComputeWaves - 1][4], pu[kComputeWaves - 1][4];
#pragma unroll
      for (int k = 1; k < kComputeWaves; ++k) {
        const float* ro = red + (w + nsub * (k < S ? k : 0)) * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = (lane >> 4) + 4 * j;
          pv[k - 1][j] = ro[row * 16 + n];
          pu[k - 1][j] = gu ? ro[(row + 8) * 16 + n] : 0.f;
        }
      }
#pragma unroll
      for (int k = 1; k < kComputeWaves; ++k) {
        if (k >= S) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sval[j] += pv[k - 1][j];
          sup[j] += pu[k - 1][j];
        }
      }
    }
  }
  // epilogue targets and the RMS scales of this lane's sequences, once
  const EpiCtx epi = make_epi(A, t);
  float rmsv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = (lane >> 4) + 4 * j;
    rmsv[j] = n < kMaxBatch ? c->rms[n] : 0.f;
  }
  rmark(2);
  auto owned_values = [&](int i, float (&val)[4], float (&up)[4]) {
    if (S > 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        val[j] = sval[j];
        up[j] = sup[j];
      }
    } else {
      tile_values(i, val, up);
    }
  };
  const int nepi = lead ? nown : 0;  // owned sub-tiles whose epilogue this wave runs
  if (publish) {
    // K-split piece ks of nks: every owned sub-tile's partial tile goes to its
    // slot (sub-tile u, piece ks) with the lowest bit of every word set (the
    // finisher's validity flag), lane-major: lane l's 16 bytes are its values
    // for (row l & 15, sequences l / 16 + 4 j)
    float* const pbase = A->part + (size_t)t.layer * A->part_blocks * 1024;
    static_for<TPW>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if (i >= nepi) return false;
      float val[4], up[4];
      owned_values(i, val, up);
      const int u = t.row0 / 16 + msub + kComputeWaves * i;
      const uint32_t off = (uint32_t)((((uint32_t)t.part_slot + (uint32_t)u * t.nks + t.ks) * 256u + 4u * lane) * 4u);
      co_store16(pbase, off, u32x4{tagged(val[0], 1u), tagged(val[1], 1u), tagged(val[2], 1u), tagged(val[3], 1u)});
      return true;
    });
  } else if (t.nks > 1) {
    // split K over nks pieces on consecutive CUs (one sub-tile per leading
    // wave, nsub <= 4).  Pieces 1.. publish their partial tiles into this
    // layer's slots with the lowest bit of every word set; piece 0 polls the
    // slots, adds the partials to its own in piece order, clears the slots
    // (it is their only reader; the next write is a step later) and runs the
    // epilogue.
    const bool own = nepi > 0;
    float val[4] = {0.f, 0.f, 0.f, 0.f}, up[4] = {0.f, 0.f, 0.f, 0.f};
    if (own) owned_values(0, val, up);
    float* const pl = A->part + ((size_t)t.layer * A->part_blocks + t.part_slot) * 1024 + w * 256;
    if (own && t.ks > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        co_store_tag(pl, (uint32_t)(((size_t)t.ks * 1024 + ((lane >> 4) + 4 * j) * 16 + row) * 4), val[j], 1u);
    }
    if (own && t.ks == 0) {
      // every piece's partial in flight at once (up to kSumBatch pieces per
      // round); for gate/up, lane ^ 8 holds the up row of a gate row and
      // hands it over by a DPP move
      constexpr int kSumBatch = 8;
      const bool gu = t.stage == ST_GU;
      // analysis builds: piece-0 wait for the other pieces (DOWN: stats word 30, others 31)
      uint64_t* psp = (MK_PHASE_TRACE && A->trace && w == 0 && lane == 0) ? MK_PSTAT(c, t.stage == ST_DOWN ? 30 : 31) : nullptr;
      const uint64_t tp0 = psp ? now_ticks() : 0;
      for (int k0 = 1; k0 < t.nks; k0 += kSumBatch) {
        uint32_t pv[kSumBatch][4];
        Spin sp = spin_start();
        for (;;) {
#pragma unroll
          for (int u = 0; u < kSumBatch; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t e = (uint32_t)((k0 + u) * 1024 + ((lane >> 4) + 4 * j) * 16 + row);
              pv[u][j] = k0 + u < t.nks ? co_load4(pl, e * 4) : 1u;
            }
          uint32_t flags = 1u;
#pragma unroll
          for (int u = 0; u < kSumBatch; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) flags &= pv[u][j];
          if (__all((flags & 1u) != 0)) break;
          if (!poll_ok(A, c, sp)) return false;
        }
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) {
          if (k0 + u >= t.nks) break;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            co_store4(pl, (uint32_t)(((size_t)(k0 + u) * 1024 + ((lane >> 4) + 4 * j) * 16 + row) * 4), 0u);
            const float pf = __uint_as_float(untag(pv[u][j]));
            val[j] += pf;
            if (gu) up[j] += dpp_f<kDppRor8>(pf);  // wave-uniform: every lane runs the move
          }
        }
      }
      if (psp) trace_add(psp, now_ticks() - tp0);
      const int lr0 = tile_row0(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) gemv_epilogue(epi, c, lr0 + row, row, (lane >> 4) + 4 * j, val[j], up[j], resid[0][j], nwv[0], rmsv[j]);
    }
  } else {
    // analysis builds: LM-head epilogue split into tile reduction / epilogue
    uint64_t* lsp = (MK_PHASE_TRACE && gst && t.stage == ST_LM) ? MK_PSTAT(c, 40) : nullptr;
    uint64_t tl0 = lsp ? now_ticks() : 0;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (i >= nepi) break;
      float val[4], up[4];
      if constexpr (NB > 0) {
        owned_values(i, val, up);
      } else {
        // the accumulator array is indexed by constants only
        static_for<TPW>([&](auto I) {
          if (decltype(I)::value == i) owned_values(decltype(I)::value, val, up);
          return true;
        });
      }
      const int lr0 = tile_row0(i);
      static_assert(kResidTiles == 2, "prefetched tiles are selected by constant index");
      const float nw = i == 0 ? nwv[0] : (i == 1 ? nwv[1] : ((has_resid && lr0 + row < M) ? bf2f(nwp[lr0 + row]) : 0.f));
      float rs[4];
      if (i < kResidTiles) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] = i == 0 ? resid[0][j] : resid[1][j];
      } else if (has_resid) {
        // residuals of tiles past the prefetched ones, polled for their tags
        const uint32_t tags = A->rowtag;
        Spin sp = spin_start();
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = (lane >> 4) + 4 * j;
            const bool need = n < A->b && lr0 + row < M;
            rs[j] = need ? co_loadf(hin, (uint32_t)(((size_t)n * A->d + lr0 + row) * 4)) : 0.f;
            if (need) ok = ok & tag_ok(__float_as_uint(rs[j]), (tags >> n) & 1u);
          }
          if (__all(ok)) break;
          if (!poll_ok(A, c, sp)) return false;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] = untagf(rs[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] = 0.f;
      }
      if (lsp) {
        const uint64_t tn = now_ticks();
        trace_add(lsp, tn - tl0);
        tl0 = tn;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) gemv_epilogue(epi, c, lr0 + row, row, (lane >> 4) + 4 * j, val[j], up[j], rs[j], nw, rmsv[j]);
      if (lsp) {
        const uint64_t tn = now_ticks();
        trace_add(lsp + 1, tn - tl0);
        tl0 = tn;
      }
    }
  }
  rmark(3);
  gmark(2);
  if (t.flags & kTaskSignal) {
    // the last task of its stage on this CU.  Consumers poll the tagged
    // outputs, so only the LM head counts its completed tasks (for the
    // greedy tokens).
    const bool lm = t.stage == ST_LM;
    if (lm) wait_mem();
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    s.synced = 1;
    if (lm && w == 0) {
      if (lane < A->b) {
        // fold this CU's argmax keys into the global ones
        const unsigned long long key = c->lmkey[lane];
        if (key) __hip_atomic_fetch_max(keys_ptr(A) + lane, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_mem();
      }
      if (lane == 0) signal_counter(A, t.signal_ctr, cu);
    }
  }
  gmark(3);
#if MK_PHASE_TRACE
  if (gst) {
    c->ppack = gpack | ((uint64_t)(c->npoll & 0xFFFF) << 48);
    c->npoll = 0;
  }
#endif
  if (A->trace) s.t_epi += now_ticks() - te0;
  return true;
}

// ---- K-split finish: for this CU's share of a K-split stage's sub-tiles,
//      poll the nks published pieces of each sub-tile, sum them in piece
//      order (a fixed order, so results do not depend on timing), clear the
//      slots (their only reader; the next write is a step later) and run the
//      stage's epilogue on the sums.  Compute wave w takes sub-tiles w, w+4, ...
#ifndef MK_FIN_BATCH
#define MK_FIN_BATCH 16
#endif
constexpr int kFinBatch = MK_FIN_BATCH;  // pieces polled per batch, every load in flight
__device__ __noinline__ bool fin_task(DArgs A, TaskP tp, int cu, int w, int lane) {
  A = uni(A);
  cu = __builtin_amdgcn_readfirstlane(cu);  // wave-uniform: scalar loads, no vmcnt drain
  w = __builtin_amdgcn_readfirstlane(w);
  Ctrl* c = ctrl_block(A);
  CState& s = c->cs[w];
  const Task t = load_task(uni(tp));
  const int M = stage_M(A, t.stage);
  const int row = lane & 15;
  const uint32_t tags = A->rowtag;
  // RMS scales of a normalised stage (one batch of loads per wave), written
  // once every compute wave is done with the previous task's scales
  const float* ss = stage_ss(A, t.stage, t.layer);
  if (ss && !(s.r_stage == t.stage && s.r_layer == t.layer)) {
    if (!s.synced && !cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    s.synced = 0;
    uint32_t none[kSsLoads] = {};
    if (!rms_scales(A, c, ss, w, lane, tags, none, false)) return false;
    s.r_stage = t.stage;
    s.r_layer = t.layer;
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
  }
  const EpiCtx epi = make_epi(A, t);
  float rmsv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = (lane >> 4) + 4 * j;
    rmsv[j] = n < kMaxBatch ? c->rms[n] : 0.f;
  }
  const bool has_resid = t.stage == ST_O || t.stage == ST_DOWN;
  const bool gu = t.stage == ST_GU;
  const float* hin = t.stage == ST_DOWN ? A->hmid + (size_t)t.layer * A->bcap * A->d
                                        : A->hres + (size_t)t.layer * A->bcap * A->d;
  const uint16_t* nwp = nullptr;
  if (t.stage == ST_O) nwp = as_const(A->layers)[t.layer].mlp_norm;
  if (t.stage == ST_DOWN) nwp = t.layer + 1 < A->L ? as_const(A->layers)[t.layer + 1].attn_norm : A->final_norm;
  float* const pbase = A->part + (size_t)t.layer * A->part_blocks * 1024;
  const int nks = t.nks;
  for (int k = w; k < t.nsub; k += kComputeWaves) {
    const int u = t.row0 / 16 + k;
    const int lr = 16 * u + row;
    // the piece values of this lane (rows lane & 15); for gate/up, lane ^ 8
    // holds the up row of a gate row (8 rows further in the tile) and hands
    // it over by a DPP move after the loads; the residuals of O / down in
    // flight with the first batch
    const uint32_t slot0 = (uint32_t)t.part_slot + (uint32_t)u * nks;
    float val[4] = {0.f, 0.f, 0.f, 0.f}, up[4] = {0.f, 0.f, 0.f, 0.f}, rs[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < nks; p0 += kFinBatch) {
      u32x4 pv[kFinBatch];
      Spin sp = spin_start();
      for (;;) {
#pragma unroll
        for (int q = 0; q < kFinBatch; ++q) {
          const bool ok = p0 + q < nks;
          const uint32_t base = (slot0 + (uint32_t)(p0 + q)) * 1024u;
          pv[q] = ok ? co_load16(pbase, base + 16u * lane) : u32x4{1u, 1u, 1u, 1u};
        }
        bool rok = true;
        if (has_resid && p0 == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = (lane >> 4) + 4 * j;
            const bool need = n < A->b && lr < M;
            rs[j] = need ? co_loadf(hin, (uint32_t)(((size_t)n * A->d + lr) * 4)) : 0.f;
            if (need) rok = rok & tag_ok(__float_as_uint(rs[j]), (tags >> n) & 1u);
          }
        }
        uint32_t flags = 1u;
#pragma unroll
        for (int q = 0; q < kFinBatch; ++q) flags &= pv[q].x & pv[q].y & pv[q].z & pv[q].w;
        if (__all(rok && (flags & 1u) != 0)) break;
        if (!poll_ok(A, c, sp)) return false;
      }
#pragma unroll
      for (int q = 0; q < kFinBatch; ++q) {
        if (p0 + q >= nks) break;
        co_store16(pbase, (slot0 + (uint32_t)(p0 + q)) * 1024u + 16u * lane, u32x4{0u, 0u, 0u, 0u});
        const u32x4 a = untag4(pv[q]);
        val[0] += __uint_as_float(a.x);
        val[1] += __uint_as_float(a.y);
        val[2] += __uint_as_float(a.z);
        val[3] += __uint_as_float(a.w);
        if (gu) {  // wave-uniform: every lane runs the moves
          up[0] += dpp_f<kDppRor8>(__uint_as_float(a.x));
          up[1] += dpp_f<kDppRor8>(__uint_as_float(a.y));
          up[2] += dpp_f<kDppRor8>(__uint_as_float(a.z));
          up[3] += dpp_f<kDppRor8>(__uint_as_float(a.w));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) rs[j] = untagf(rs[j]);
    const float nw = (has_resid && lr < M) ? bf2f(nwp[lr]) : 0.f;
    if (!gu) {
#pragma unroll
      for (int j = 0; j < 4; ++j) up[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) gemv_epilogue(epi, c, lr, row, (lane >> 4) + 4 * j, val[j], up[j], rs[j], nw, rmsv[j]);
  }
  if (t.flags & kTaskSignal) {
    // the LM head's last finish task on this CU: fold the CU's argmax keys
    // into the global ones and count the task (for the greedy tokens)
    wait_mem();
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    s.synced = 1;
    if (w == 0) {
      if (lane < A->b) {
        const unsigned long long key = c->lmkey[lane];
        if (key) __hip_atomic_fetch_max(keys_ptr(A) + lane, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_mem();
      }
      if (lane == 0) signal_counter(A, t.signal_ctr, cu);
    }
  }
  return true;
}

// ---- embedding gather: h0 = E[token] for 64 columns, plus the first
//      RMSNorm's input and per-16-column sums of squares.
__device__ __noinline__ bool embed_task(DArgs A, TaskP tp, int cu, int w, int lane) {
  A = uni(A);
  cu = __builtin_amdgcn_readfirstlane(cu);  // wave-uniform: scalar loads, no vmcnt drain
  w = __builtin_amdgcn_readfirstlane(w);
  Ctrl* c = ctrl_block(A);
  CState& s = c->cs[w];
  const Task t = load_task(uni(tp));
  const int tid = w * 64 + lane, n = tid >> 4, col = t.row0 + 4 * (tid & 15);
  float h[4] = {0.f, 0.f, 0.f, 0.f};
  const bool valid = n < A->b;
  const uint32_t tg = (A->rowtag >> n) & 1u;
  if (valid) {
    const uint16_t* e = A->embed + (size_t)c->tok[n] * A->d + col;
    u32x2 ev = *(const u32x2*)e;
    h[0] = bf_lo(ev.x); h[1] = bf_hi(ev.x); h[2] = bf_lo(ev.y); h[3] = bf_hi(ev.y);
    const uint16_t* nw = as_const(A->layers)[0].attn_norm + col;
    co_store16(A->hres, (uint32_t)(((size_t)n * A->d + col) * 4),
               u32x4{tagged(h[0], tg), tagged(h[1], tg), tagged(h[2], tg), tagged(h[3], tg)});
    if (A->dump) *(f32x4*)(A->dump + (size_t)n * A->d + col) = f32x4{h[0], h[1], h[2], h[3]};
    co_store16(A->xattn, (uint32_t)(((size_t)n * A->d + col) * 4),
               u32x4{tagged(h[0] * bf2f(nw[0]), tg), tagged(h[1] * bf2f(nw[1]), tg),
                     tagged(h[2] * bf2f(nw[2]), tg), tagged(h[3] * bf2f(nw[3]), tg)});
  }
  float ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  if (valid && (tid & 3) == 0) co_store_tag(A->ssattn, (uint32_t)((((size_t)col >> 4) * A->bcap + n) * 4), ss, tg);
  // consumers poll the tagged words: no completion wait, no counter
  if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
  s.synced = 1;
  return true;
}

// ---- attention --------------------------------------------------------
// 2^x with the hardware instruction (about 1 ulp on normal results, 0 for
// x = -inf, results below the normal range flush to 0: softmax weights that
// small do not change a sum that holds a weight of 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct SoftState {
  float m, l;
};

// A head's 8 own elements (a0, a1: elements e0..e0+7) and their 8
// rotate-half partners (b0, b1) of a raw q/k row: apply the optional per-head
// RMSNorm and RoPE at position p.
template <int HD>
__device__ __forceinline__ void rope_head(DArgs A, u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, const uint16_t* normw, int p,
                                          int e0, float* out) {
  constexpr int LPR = HD / 8;
  const int pe = (e0 + HD / 2) % HD;
  float x[8] = {__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z), __uint_as_float(a0.w),
                __uint_as_float(a1.x), __uint_as_float(a1.y), __uint_as_float(a1.z), __uint_as_float(a1.w)};
  float y[8] = {__uint_as_float(b0.x), __uint_as_float(b0.y), __uint_as_float(b0.z), __uint_as_float(b0.w),
                __uint_as_float(b1.x), __uint_as_float(b1.y), __uint_as_float(b1.z), __uint_as_float(b1.w)};
  if (normw) {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
    const float rs = 1.0f / sqrtf(ss / (float)HD + A->eps);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      x[u] = x[u] * rs * bf2f(normw[e0 + u]);
      y[u] = y[u] * rs * bf2f(normw[pe + u]);
    }
  }
  const bool first = e0 < HD / 2;
  const int fi = first ? e0 : e0 - HD / 2;
  const float* cs = A->rope + ((size_t)p * (HD / 2) + fi) * 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float cv = cs[2 * u], sv = cs[2 * u + 1];
    out[u] = first ? x[u] * cv - y[u] * sv : x[u] * cv + y[u] * sv;
  }
}

// One attention task: this CU's range of the flattened (sequence, KV head,
// position) rows, as pieces that each lie inside one (sequence, KV head)
// segment.  Scores of a chunk come from MFMAs (the group's query heads as A,
// bf16 hi + lo halves; the chunk's K rows as B), the softmax state (m, l) per
// head is wave-uniform with one rescale per chunk, and V is accumulated on
// the VALU with each lane group holding 8 dimensions of its rows.  The four
// waves' states merge in LDS (wave h merges head h); a piece that is a whole
// segment stores the output, otherwise it publishes its partial and the last
// piece to arrive merges the segment.
template <int HD, int GM>
__device__ __noinline__ bool attn_task(DArgs A, TaskP tp, int cu, int w, int lane) {
  static_assert(GM <= 8, "at most 8 query heads per KV head");
  A = uni(A);
  cu = __builtin_amdgcn_readfirstlane(cu);  // wave-uniform: scalar loads, no vmcnt drain
  w = __builtin_amdgcn_readfirstlane(w);
  char* ring = mk_lds;
  Ctrl* c = ctrl_block(A);
  CState& s = c->cs[w];
  const Task t = load_task(uni(tp));
  constexpr int LPR = HD / 8, RP = 64 / LPR, RPC = 4096 / HD, NP = RPC / RP;
  constexpr int NRB = RPC / 16;        // 16-row blocks per chunk (MFMA N)
  constexpr int NDS = HD / 32;         // 32-wide steps over the head dimension (MFMA K)
  constexpr int SW = HD + 4;           // floats per head in a state / partial record
  constexpr float kLog2e = 1.4426950408889634f;
  const int l = t.layer, G = A->G, e0 = (lane % LPR) * 8, gi = lane / LPR;
  const int r16 = lane & 15, lr = lane >> 4;  // MFMA output layout: row r16 of a block, heads 4 lr + i
  const float qscale = kLog2e / sqrtf((float)HD);
  const long long W0 = attn_total(c, A->b, A->nkv);
  // this CU's slot: pieces, partial slots and the finisher role go by slot
  const int nacu = attn_nacu(A, t.layer, W0), slot = attn_slot(A, t.layer, cu);
  const int pad = attn_pad_rows(A, W0, nacu);
  const long long W = attn_padded(A, W0, pad);  // flattened (padded) length: all positions below are in it
  long long pos = slot < nacu ? cu_lo(slot, W, nacu) : W, hi = slot < nacu ? cu_lo(slot + 1, W, nacu) : W;
  Piece P;
  int qc = s.q, pidx = 0;
  const MK_AS4 LayerW& lw = as_const(A->layers)[l];
  // staging-buffer layout while attention runs: wave states (2 piece
  // parities x 4 waves x GM x SW), the batch's scaled queries
  // (kAttnBatch x GM x HD), its new K and V rows (kAttnBatch x 2 x HD), then
  // per wave the chunk's transposed probabilities
  float* stb = (float*)xb_stage(A);
  const int stride_st = kComputeWaves * GM * SW;
  float* qs = stb + 2 * stride_st;
  float* knv = qs + kAttnBatch * GM * HD;
  constexpr int GMP = GM <= 4 ? 4 : 8;  // heads per probability row (the group padded to 4 or 8)
  float* pb = knv + kAttnBatch * 2 * HD + w * RPC * GMP;  // P: 2 planes x RPC rows x GMP heads, bf16
  const float* qkv_l = A->qkv + (size_t)l * A->bcap * A->nqkv;
  const uint32_t tags = A->rowtag;
  // the staging buffer is rewritten below (queries, new rows, wave states):
  // every compute wave must be done with the previous task's use of it
  if (!s.synced && !cbar(A, c, s.gen, lane, &s.w_bar)) return false;
  s.synced = 0;
  // trace: attention phase totals of compute wave 0 (per-CU stats words 32..41)
  uint64_t* ast = (MK_PHASE_TRACE && A->trace && w == 0 && lane == 0) ? MK_PSTAT(c, 0) : nullptr;
  uint64_t tlast = ast ? now_ticks() : 0;
  // per-task offsets (analysis trace word 2): queries ready, pieces done, finish done
  const uint64_t at0 = tlast;
  uint64_t apack = 0;
  auto amark = [&](int k) {
    if (ast && !((apack >> (16 * k)) & 0xFFFF)) apack |= ((now_ticks() - at0) & 0xFFFF) << (16 * k);
  };
  auto mark = [&](int k) {
    if (ast) {
      const uint64_t tn = now_ticks();
      trace_add(ast + k, tn - tlast);
      tlast = tn;
    }
  };
  auto bcast = [](float v, int src_lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
  };
  // The finisher of a segment split over several CUs is the CU holding its
  // first rows.  Pieces publish their partials (o, m, l per head) into
  // per-layer slots with the lowest mantissa bit of every word set; the
  // finisher polls the slots until every word is set, merges, stores the
  // output and clears the slots (it is their only reader, and the next write
  // of a slot is in a later step).  Compute wave w merges heads w, w + 4;
  // LPP lanes cover one piece's head vector, PPI pieces per pass; all loads
  // of a pass are issued before any is used.
  struct Pend {
    int sid, npieces, c_first, i, g;
    long long seg_start;
  };
  const int pstride = GM * SW;
  float* const apart_l = A->apart + (size_t)l * (A->ncu + A->bcap * A->nkv) * pstride;
  auto finish_segment = [&](const Pend& pd) -> bool {
    const int sid = pd.sid, npieces = pd.npieces, c_first = pd.c_first;
    const long long seg_start = pd.seg_start;
    float* ob = A->attn_out + ((size_t)l * A->bcap + pd.i) * A->qdim + (size_t)pd.g * G * HD;
    constexpr int LPP = HD / 4, PPI = 64 / LPP, kMergeIt = 16;
    const int sub = lane / LPP, el = (lane % LPP) * 4;
    // byte offset of piece pc's record from the layer's (wave-uniform) slot
    // base: per-lane offsets keep every access a single buffer instruction
    auto piece_off = [&](int pc) -> uint32_t {
      const int pcu = W >= nacu ? c_first + pc : cu_of(seg_start + pc, W, nacu);
      return (uint32_t)(pcu + sid) * (uint32_t)(pstride * 4);
    };
    for (int h = w; h < G; h += kComputeWaves) {
      float Mrun = -INFINITY, Lrun = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int p0 = 0; p0 < npieces; p0 += PPI * kMergeIt) {
        u32x4 ov[kMergeIt];
        u32x2 ml[kMergeIt];
        uint32_t po[kMergeIt];
#pragma unroll
        for (int k = 0; k < kMergeIt; ++k) {
          const int pc = p0 + k * PPI + sub;
          po[k] = piece_off(pc < npieces ? pc : 0);
        }
        Spin sp = spin_start();
        const uint64_t tp0 = MK_PHASE_TRACE && ast ? now_ticks() : 0;
        for (;;) {
          if (MK_PHASE_TRACE && ast) trace_add(MK_PSTAT(c, 46), 1);
#if MK_PHASE_TRACE
          if (ast) c->npoll += 1;
#endif
          // every load of the pass in flight before any flag is tested
#pragma unroll
          for (int k = 0; k < kMergeIt; ++k) {
            ov[k] = co_load16(apart_l, po[k] + (uint32_t)((h * SW + el) * 4));
            ml[k] = co_load8(apart_l, po[k] + (uint32_t)((h * SW + HD) * 4));
          }
          uint32_t flags = 1u;
#pragma unroll
          for (int k = 0; k < kMergeIt; ++k) {
            const uint32_t f = ov[k].x & ov[k].y & ov[k].z & ov[k].w & ml[k].x & ml[k].y;
            flags &= p0 + k * PPI + sub < npieces ? f : 1u;
          }
          if (__all((flags & 1u) != 0)) break;
          if (!poll_ok(A, c, sp)) return false;
        }
        if (MK_PHASE_TRACE && ast) trace_add(MK_PSTAT(c, 47), now_ticks() - tp0);
        float m2[kMergeIt], l2[kMergeIt];
#pragma unroll
        for (int k = 0; k < kMergeIt; ++k) {
          const int pc = p0 + k * PPI + sub;
          if (pc < npieces) {
            co_store16(apart_l, po[k] + (uint32_t)((h * SW + el) * 4), u32x4{0u, 0u, 0u, 0u});
            if (el == 0) co_store8(apart_l, po[k] + (uint32_t)((h * SW + HD) * 4), u32x2{0u, 0u});
          }
          ov[k] = untag4(ov[k]);
          m2[k] = pc < npieces ? __uint_as_float(untag(ml[k].x)) : -INFINITY;
          l2[k] = __uint_as_float(untag(ml[k].y));
        }
        float mb = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMergeIt; ++k) mb = fmaxf(mb, m2[k]);
        mb = group_max<16>(mb);
        mb = swap16_max(mb);
        mb = swap32_max(mb);
        const float mn = fmaxf(Mrun, mb);
        const float fr = Mrun == -INFINITY ? 0.f : exp2f(Mrun - mn);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] *= fr;
        Lrun *= fr;
#pragma unroll
        for (int k = 0; k < kMergeIt; ++k) {
          const float f = m2[k] == -INFINITY ? 0.f : exp2f(m2[k] - mn);
          acc[0] += f * __uint_as_float(ov[k].x);
          acc[1] += f * __uint_as_float(ov[k].y);
          acc[2] += f * __uint_as_float(ov[k].z);
          acc[3] += f * __uint_as_float(ov[k].w);
          Lrun += f * l2[k];
        }
        Mrun = mn;
      }
#pragma unroll
      for (int msk = LPP; msk < 64; msk <<= 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += __shfl_xor(acc[u], msk);
        Lrun += __shfl_xor(Lrun, msk);
      }
      if (sub == 0) {
        const float inv = 1.0f / Lrun;
        const uint32_t tg = (tags >> pd.i) & 1u;
        co_store16(ob, (uint32_t)((h * HD + el) * 4),
                   u32x4{tagged(acc[0] * inv, tg), tagged(acc[1] * inv, tg), tagged(acc[2] * inv, tg),
                         tagged(acc[3] * inv, tg)});
      }
    }
    if (ast) trace_add(ast + 8, 1);
    return true;
  };
  Pend pend{};
  bool has_pend = false;
  // analysis builds: sub-phases of the query preparation (compute wave 0)
  uint64_t* qsp = ast ? MK_PSTAT(c, 32) : nullptr;
  uint64_t tq = qsp ? now_ticks() : 0;
  auto qmark = [&](int k) {
    if (qsp) {
      const uint64_t tn = now_ticks();
      trace_add(qsp + k, tn - tq);
      tq = tn;
    }
  };
  long long bpos = pos;
  while (bpos < hi) {
    // ---- a batch of up to kAttnBatch pieces: first every query row (QK-norm,
    // RoPE, scale) and every new K row (QK-norm, RoPE) and V row of the batch,
    // one row per lane group, all loads in flight together; the new rows are
    // rounded to bf16 and written to the cache here
    int bi[kAttnBatch], bg[kAttnBatch], bnew[kAttnBatch], nbp = 0;
    {
      long long tpos = bpos;
      Piece Q;
#pragma unroll
      for (int k = 0; k < kAttnBatch; ++k) {
        bi[k] = bg[k] = bnew[k] = 0;
        if (next_piece(c, A->b, A->nkv, RPC, pad, tpos, hi, Q)) {
          bi[k] = Q.i;
          bg[k] = Q.g;
          bnew[k] = Q.has_new;
          nbp = k + 1;
        }
      }
    }
    // the rest of the range is segment padding: no piece left (uniform
    // over the compute waves, before any barrier of the batch)
    if (nbp == 0) break;
    const int nrows = nbp * (GM + 1);  // rows (piece, h): h < GM queries, h == GM the new K / V
    qmark(0);
    for (int r0 = 0; r0 < nrows; r0 += kComputeWaves * RP) {
      const int r = r0 + w * RP + gi;
      const int k = r / (GM + 1), h = r - k * (GM + 1);
      int pi = bi[0], pg = bg[0], pn = bnew[0];
#pragma unroll
      for (int kk = 1; kk < kAttnBatch; ++kk)
        if (k == kk) {
          pi = bi[kk];
          pg = bg[kk];
          pn = bnew[kk];
        }
      const bool is_k = h == GM;
      const bool valid = r < nrows && (is_k ? pn != 0 : h < G);
      const int pp = c->slen[pi] - 1;
      const uint32_t rowoff = (uint32_t)pi * A->nqkv;
      const uint32_t off = valid ? rowoff + (is_k ? A->qdim + pg * HD : (pg * G + h) * HD) : 0u;
      const uint32_t voff = valid && is_k ? rowoff + A->qdim + A->kvdim + pg * HD : 0u;
      // the head's elements, their rotate-half partners and (new rows) the V
      // row, loaded again until every word carries the sequence's step tag
      const int pe = (e0 + HD / 2) % HD;
      const uint32_t tg = (tags >> pi) & 1u;
      u32x4 a0, a1, b0, b1, v0, v1;
      {
        Spin sp = spin_start();
        for (;;) {
          a0 = co_load16(qkv_l, (off + e0) * 4);
          a1 = co_load16(qkv_l, (off + e0 + 4) * 4);
          b0 = co_load16(qkv_l, (off + pe) * 4);
          b1 = co_load16(qkv_l, (off + pe + 4) * 4);
          v0 = co_load16(qkv_l, (voff + e0) * 4);
          v1 = co_load16(qkv_l, (voff + e0 + 4) * 4);
          const bool ok = !valid || (tag_ok4(a0, tg) & tag_ok4(a1, tg) & tag_ok4(b0, tg) & tag_ok4(b1, tg) &
                                     (!is_k || (tag_ok4(v0, tg) & tag_ok4(v1, tg))));
          if (__all(ok)) break;
          if (!poll_ok(A, c, sp)) return false;
        }
        a0 = untag4(a0);
        a1 = untag4(a1);
        b0 = untag4(b0);
        b1 = untag4(b1);
        v0 = untag4(v0);
        v1 = untag4(v1);
      }
      float x8[8];
      rope_head<HD>(A, a0, a1, b0, b1, A->qk_norm ? (is_k ? lw.k_norm : lw.q_norm) : nullptr, valid ? pp : 0, e0, x8);
      qmark(1);
      if (valid && !is_k) {
        float* qd = qs + ((size_t)k * GM + h) * HD + e0;
        lds_st16((char*)qd, u32x4{__float_as_uint(x8[0] * qscale), __float_as_uint(x8[1] * qscale),
                                  __float_as_uint(x8[2] * qscale), __float_as_uint(x8[3] * qscale)});
        lds_st16((char*)(qd + 4), u32x4{__float_as_uint(x8[4] * qscale), __float_as_uint(x8[5] * qscale),
                                        __float_as_uint(x8[6] * qscale), __float_as_uint(x8[7] * qscale)});
      }
      if (valid && is_k) {
        const u32x4 kb = {pack_bf2(x8[0], x8[1]), pack_bf2(x8[2], x8[3]), pack_bf2(x8[4], x8[5]), pack_bf2(x8[6], x8[7])};
        const u32x4 vb = {pack_bf2(__uint_as_float(v0.x), __uint_as_float(v0.y)), pack_bf2(__uint_as_float(v0.z), __uint_as_float(v0.w)),
                          pack_bf2(__uint_as_float(v1.x), __uint_as_float(v1.y)), pack_bf2(__uint_as_float(v1.z), __uint_as_float(v1.w))};
        const size_t slot_row = kv_row<false>(A, l, pi, pg, pp) * HD + e0;
        *(u32x4*)(A->kc + slot_row) = kb;
        *(u32x4*)(A->vc + slot_row) = vb;
        float kf[8], vf[8];
        unpack8(kb, kf);
        unpack8(vb, vf);
        float* kd = knv + (size_t)k * 2 * HD + e0;
        lds_st16((char*)kd, u32x4{__float_as_uint(kf[0]), __float_as_uint(kf[1]), __float_as_uint(kf[2]), __float_as_uint(kf[3])});
        lds_st16((char*)(kd + 4), u32x4{__float_as_uint(kf[4]), __float_as_uint(kf[5]), __float_as_uint(kf[6]), __float_as_uint(kf[7])});
        lds_st16((char*)(kd + HD), u32x4{__float_as_uint(vf[0]), __float_as_uint(vf[1]), __float_as_uint(vf[2]), __float_as_uint(vf[3])});
        lds_st16((char*)(kd + HD + 4), u32x4{__float_as_uint(vf[4]), __float_as_uint(vf[5]), __float_as_uint(vf[6]), __float_as_uint(vf[7])});
      }
    }
    qmark(2);
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    qmark(3);
    amark(0);
    for (int bk = 0; bk < nbp; ++bk) {
    next_piece(c, A->b, A->nkv, RPC, pad, bpos, hi, P);
    if (ast) trace_add(ast + 7, 1);
    const float* qk = qs + (size_t)bk * GM * HD;  // this piece's scaled queries
    float* sb = stb + (pidx & 1) * stride_st + w * GM * SW;  // this wave's state of the piece
    if constexpr (GM == 1) {
      // One query head per KV head: an MFMA tile would use one of its 16 rows,
      // so the VALU does it.  Lane l takes K/V row l / LPV of every chunk and
      // the 64 dims (l % LPV) * 64 .. + 63; the loader stored row r's 16-byte
      // groups rotated by r & 7 (attn_rot), so the lanes of one LDS access
      // fall in different banks while each lane keeps fixed dims.  Scores:
      // v_dot2 of the bf16 K row with q as bf16 hi + lo; softmax state
      // wave-uniform; P.V accumulates each lane's row in fp32 and the rows are
      // summed across lanes once per piece.
      constexpr int LPV = HD / 64;  // lanes per row
      constexpr int GPR = HD / 8;   // 16-byte groups per row
      static_assert(64 / LPV == RPC, "one row per lane group per chunk");
      const int vrow = lane / LPV, hh = lane % LPV, rot = vrow & 7;
      uint32_t goff[8];  // byte offset of this lane's group i inside its row
#pragma unroll
      for (int i = 0; i < 8; ++i) goff[i] = (uint32_t)((((hh * 8 + i) - rot) & (GPR - 1)) * 16);
      u32x4 qh[8], ql[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const char* src = (const char*)(qk + hh * 64 + i * 8);
        split8(lds_ld16(src), lds_ld16(src + 16), qh[i], ql[i]);
      }
      float o[64];
#pragma unroll
      for (int d = 0; d < 64; ++d) o[d] = 0.f;
      float m1 = -INFINITY, l1 = 0.f;
      mark(0);
      for (int ch = 0; ch < P.nch; ++ch) {
        const int gq = qc + ch;
        if ((gq & (kComputeWaves - 1)) != w) continue;
        const uint64_t tw0 = MK_PHASE_TRACE && ast ? now_ticks() : 0;
        if (!wait_chunk(A, c, gq, s.w_empty)) return false;
        if (MK_PHASE_TRACE && ast) trace_add(ast + 9, now_ticks() - tw0);
        const char* slot = ring + (size_t)(gq % A->nslot) * kSlotBytes;
        const int rows = min(RPC, P.ncached - ch * RPC);
        const char* kr = slot + (size_t)vrow * HD * 2;
        float sc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 kv = lds_ld16(kr + goff[i]);
          sc = dot8_bf16(kv, qh[i], dot8_bf16(kv, ql[i], sc));
        }
        if constexpr (LPV == 2) sc += dpp_f<kDppXor1>(sc);
        sc = vrow < rows ? sc : -INFINITY;
        float mx = group_max<16>(sc);
        mx = swap16_max(mx);
        mx = swap32_max(mx);
        const float mnew = fmaxf(m1, mx);  // finite: every chunk has a row
        const float fa = fast_exp2(m1 - mnew);
        const float pv = fast_exp2(sc - mnew);  // 0 for rows past the chunk
        float ps = hh == 0 ? pv : 0.f;
        ps = group_sum<16>(ps);
        ps = swap16_sum(ps, ps);
        ps = swap32_sum(ps, ps);
        l1 = l1 * fa + ps;
        if (fa != 1.f) {
#pragma unroll
          for (int d = 0; d < 64; ++d) o[d] *= fa;
        }
        m1 = mnew;
        const char* vr = slot + 8192 + (size_t)vrow * HD * 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float vf[8];
          unpack8(lds_ld16(vr + goff[i]), vf);
#pragma unroll
          for (int u = 0; u < 8; ++u) o[i * 8 + u] += pv * vf[u];
        }
        free_chunk(A, c, gq, lane);
      }
      // the new row (K, V rounded to bf16, already in the cache), absorbed by
      // wave 0: every lane forms the score from its own dims, row 0's lanes
      // take p * v
      if (w == 0 && P.has_new) {
        const float* kd = knv + (size_t)bk * 2 * HD;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 qa = lds_ld16((const char*)(qk + hh * 64 + i * 8)), qb = lds_ld16((const char*)(qk + hh * 64 + i * 8 + 4));
          const u32x4 ka = lds_ld16((const char*)(kd + hh * 64 + i * 8)), kb = lds_ld16((const char*)(kd + hh * 64 + i * 8 + 4));
          part += __uint_as_float(qa.x) * __uint_as_float(ka.x) + __uint_as_float(qa.y) * __uint_as_float(ka.y) +
                  __uint_as_float(qa.z) * __uint_as_float(ka.z) + __uint_as_float(qa.w) * __uint_as_float(ka.w) +
                  __uint_as_float(qb.x) * __uint_as_float(kb.x) + __uint_as_float(qb.y) * __uint_as_float(kb.y) +
                  __uint_as_float(qb.z) * __uint_as_float(kb.z) + __uint_as_float(qb.w) * __uint_as_float(kb.w);
        }
        if constexpr (LPV == 2) part += dpp_f<kDppXor1>(part);
        const float mn = fmaxf(m1, part);
        const float fn = fast_exp2(m1 - mn), pn = fast_exp2(part - mn);
        l1 = l1 * fn + pn;
        m1 = mn;
        const float pr = vrow == 0 ? pn : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 va = lds_ld16((const char*)(kd + HD + hh * 64 + i * 8)), vb = lds_ld16((const char*)(kd + HD + hh * 64 + i * 8 + 4));
          const float vv[8] = {__uint_as_float(va.x), __uint_as_float(va.y), __uint_as_float(va.z), __uint_as_float(va.w),
                               __uint_as_float(vb.x), __uint_as_float(vb.y), __uint_as_float(vb.z), __uint_as_float(vb.w)};
#pragma unroll
          for (int u = 0; u < 8; ++u) o[i * 8 + u] = o[i * 8 + u] * fn + pr * vv[u];
        }
      }
      mark(1);
      // sum the rows across lanes (transposing butterfly over lane bits 5 ..
      // log2(LPV)): lane l ends with dims (l & ~(LPV-1)) .. + 64/(64/LPV) - 1
      // of its 64
#pragma unroll
      for (int k = 0; k < 32; ++k) o[k] = swap32_sum(o[k], o[k + 32]);
#pragma unroll
      for (int k = 0; k < 16; ++k) o[k] = swap16_sum(o[k], o[k + 16]);
      {
        const bool b3 = lane & 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float keep = b3 ? o[k + 8] : o[k], send = b3 ? o[k] : o[k + 8];
          o[k] = keep + dpp_f<kDppRor8>(send);  // lane ^ 8
        }
      }
      {
        const bool b2 = lane & 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float keep = b2 ? o[k + 4] : o[k], send = b2 ? o[k] : o[k + 4];
          const float s_up = b2 ? send : 0.f, s_dn = b2 ? 0.f : send;
          o[k] = keep + dpp_f<kDppShl4>(s_up) + dpp_f<kDppShr4>(s_dn);  // lane ^ 4
        }
      }
      {
        const bool b1 = lane & 2;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float keep = b1 ? o[k + 2] : o[k], send = b1 ? o[k] : o[k + 2];
          o[k] = keep + dpp_f<kDppXor2>(send);  // lane ^ 2
        }
      }
      if constexpr (LPV == 1) {
        const bool b0 = lane & 1;
        const float keep = b0 ? o[1] : o[0], send = b0 ? o[0] : o[1];
        o[0] = keep + dpp_f<kDppXor1>(send);  // lane ^ 1
        sb[lane] = o[0];
      } else {
        sb[hh * 64 + (lane & ~1)] = o[0];
        sb[hh * 64 + (lane & ~1) + 1] = o[1];
      }
      if (lane == 0) {
        sb[HD] = m1;
        sb[HD + 1] = l1;
      }
    } else {
    u32x4 qa_hi[NDS], qa_lo[NDS];
    {
      const int kq = 8 * lr;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        qa_hi[ds] = qa_lo[ds] = u32x4{0, 0, 0, 0};
        if (r16 < G) {
          const char* src = (const char*)(qk + r16 * HD + ds * 32 + kq);
          split8(lds_ld16(src), lds_ld16(src + 16), qa_hi[ds], qa_lo[ds]);
        }
      }
    }
    // output accumulators in the MFMA layout: lane holds heads 4 lr + i of
    // dims nb * 16 + r16
    constexpr int NB16 = HD / 16;  // 16-wide dim blocks (MFMA N of P.V)
    constexpr int NKS = RPC / 32;  // 32-row steps of a chunk (MFMA K of P.V)
    float mrun[GM], lrun[GM];
    f32x4 O[NB16];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      mrun[h] = -INFINITY;
      lrun[h] = 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < NB16; ++nb) O[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the value of a per-head wave-uniform array for this lane's head 4 lr + i
    auto lane_head = [&](const float (&v)[GM], int i) { return (GM > 4 && lr == 1) ? v[(4 + i) % GM] : v[i % GM]; };
    uint16_t* p_hi = (uint16_t*)pb;  // P [RPC rows][GMP heads] as bf16 hi, then lo
    uint16_t* p_lo = p_hi + RPC * GMP;
    // A operand of P.V read transposed: lane s of each 16-lane block loads
    // heads 4 min(s & 3, GMP / 4 - 1) .. + 3 of row s >> 2, so lane r16 <
    // GMP receives head r16 of 4 consecutive rows (rows past GMP repeat
    // heads; rows past the group are never stored)
    const int p_off = ((lane & 15) >> 2) * GMP + 4 * min(lane & 3, GMP / 4 - 1);
    mark(0);
    // cached rows, streamed by the loader
    for (int ch = 0; ch < P.nch; ++ch) {
      const int gq = qc + ch;
      if ((gq & (kComputeWaves - 1)) != w) continue;
      const uint64_t tw0 = MK_PHASE_TRACE && ast ? now_ticks() : 0;
      if (!wait_chunk(A, c, gq, s.w_empty)) return false;
      if (MK_PHASE_TRACE && ast) trace_add(ast + 9, now_ticks() - tw0);
      const char* slot = ring + (size_t)(gq % A->nslot) * kSlotBytes;
      const int rows = min(RPC, P.ncached - ch * RPC);
      // scores S[head][row]: lane holds heads 4 lr + i of row rb * 16 + r16
      f32x4 S[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        S[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const u32x4 kb = lds_ld16(slot + ((rb * 16 + r16) * HD + ds * 32 + 8 * lr) * 2);
          S[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa_lo[ds]),
                                                          __builtin_bit_cast(bf16x8_t, kb), S[rb], 0, 0, 0);
          S[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa_hi[ds]),
                                                          __builtin_bit_cast(bf16x8_t, kb), S[rb], 0, 0, 0);
        }
      }
      // chunk maxima per head (rows past the chunk's end are -inf)
      float mx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          S[rb][i] = rb * 16 + r16 < rows ? S[rb][i] : -INFINITY;
          m = fmaxf(m, S[rb][i]);
        }
        mx[i] = group_max<16>(m);
      }
      float mnew[GM], fa[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        mnew[h] = fmaxf(mrun[h], bcast(mx[h & 3], 16 * (h >> 2)));
        fa[h] = mnew[h] == -INFINITY ? 1.f : fast_exp2(mrun[h] - mnew[h]);
      }
      // probabilities of this lane's rows for its heads and their row sums;
      // P to LDS as bf16 hi + lo planes, a row's 4 heads in one 8-byte store
      // (the A operand of P.V)
      float mh[4], sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) mh[i] = lane_head(mnew, i);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        uint32_t ph[2] = {0u, 0u}, pl[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // masked rows hold -inf and give exp2(-inf) = 0; mh is finite
          // (every chunk has at least one row)
          const float pv = fast_exp2(S[rb][i] - mh[i]);
          sum[i] += pv;
          // hi = p truncated to bf16, lo = the remainder truncated to bf16
          // (p in [0, 1]: the pair keeps p to about 2^-16)
          const uint32_t bits = __float_as_uint(pv);
          const float rem = pv - __uint_as_float(bits & 0xFFFF0000u);
          ph[i >> 1] |= (bits >> 16) << (16 * (i & 1));
          pl[i >> 1] |= (__float_as_uint(rem) >> 16) << (16 * (i & 1));
        }
        if (4 * lr < GMP) {
          const int e = (rb * 16 + r16) * GMP + 4 * lr;
          *(u32x2*)(p_hi + e) = u32x2{ph[0], ph[1]};
          *(u32x2*)(p_lo + e) = u32x2{pl[0], pl[1]};
        }
      }
      float ls[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[i] = group_sum<16>(sum[i]);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        lrun[h] = lrun[h] * fa[h] + bcast(ls[h & 3], 16 * (h >> 2));
        mrun[h] = mnew[h];
      }
      {
        float fl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fl[i] = lane_head(fa, i);
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[nb][i] *= fl[i];
      }
      // P.V on MFMA: A = P^T rows (heads) x 32 cached rows, B = 32 V rows x
      // 16 dims of the row-major chunk, read transposed: lane s of each
      // 16-lane block loads dims 4 (s & 3) .. + 3 of row (s >> 2), so lane
      // r16 of block lr receives dim r16 of 4 consecutive rows; two reads
      // give rows r0 .. r0 + 7
      const char* vrow = slot + 8192 + (size_t)(((lane & 15) >> 2) * HD + 4 * (lane & 3)) * 2;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int r0 = ks * 32 + 8 * lr;
        const char* pa = (const char*)(p_hi + r0 * GMP + p_off);
        const u32x2 h03 = lds_ld8_tr16(pa), h47 = lds_ld8_tr16(pa + 4 * GMP * 2);
        const u32x2 l03 = lds_ld8_tr16(pa + RPC * GMP * 2), l47 = lds_ld8_tr16(pa + (RPC + 4) * GMP * 2);
        const u32x4 ah = {h03.x, h03.y, h47.x, h47.y}, al = {l03.x, l03.y, l47.x, l47.y};
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) {
          const char* vp = vrow + (size_t)(r0 * HD + nb * 16) * 2;
          const u32x2 v03 = lds_ld8_tr16(vp), v47 = lds_ld8_tr16(vp + 4 * HD * 2);
          const u32x4 bv = {v03.x, v03.y, v47.x, v47.y};
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al), __builtin_bit_cast(bf16x8_t, bv),
                                                          O[nb], 0, 0, 0);
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah), __builtin_bit_cast(bf16x8_t, bv),
                                                          O[nb], 0, 0, 0);
        }
      }
      free_chunk(A, c, gq, lane);
    }
    // the new row (K, V rounded to bf16, already in the cache), absorbed by
    // wave 0
    if (w == 0 && P.has_new) {
      const float* kd = knv + (size_t)bk * 2 * HD;
      float kn[8];
      {
        const u32x4 k0 = lds_ld16((const char*)(kd + e0)), k1 = lds_ld16((const char*)(kd + e0 + 4));
        kn[0] = __uint_as_float(k0.x); kn[1] = __uint_as_float(k0.y); kn[2] = __uint_as_float(k0.z); kn[3] = __uint_as_float(k0.w);
        kn[4] = __uint_as_float(k1.x); kn[5] = __uint_as_float(k1.y); kn[6] = __uint_as_float(k1.z); kn[7] = __uint_as_float(k1.w);
      }
      float fn[GM], pn[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        fn[h] = 1.f;
        pn[h] = 0.f;
        if (h >= G) continue;
        const float* qh = qk + h * HD + e0;
        const u32x4 qa = lds_ld16((const char*)qh), qb2 = lds_ld16((const char*)(qh + 4));
        const float qv[8] = {__uint_as_float(qa.x), __uint_as_float(qa.y), __uint_as_float(qa.z), __uint_as_float(qa.w),
                             __uint_as_float(qb2.x), __uint_as_float(qb2.y), __uint_as_float(qb2.z), __uint_as_float(qb2.w)};
        float sc = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) sc += qv[u] * kn[u];
        sc = bcast(group_sum<LPR>(sc), 0);  // every lane group computed the same row
        const float mn = fmaxf(mrun[h], sc);
        fn[h] = exp2f(mrun[h] - mn);
        pn[h] = exp2f(sc - mn);
        lrun[h] = lrun[h] * fn[h] + pn[h];
        mrun[h] = mn;
      }
      float fl[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fl[i] = lane_head(fn, i);
        pl[i] = lane_head(pn, i);
      }
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb) {
        const float vv = kd[HD + nb * 16 + r16];
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nb][i] = O[nb][i] * fl[i] + pl[i] * vv;
      }
    }
    mark(1);
    // wave state -> LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * lr + i;
      if (hh < G) {
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) sb[hh * SW + nb * 16 + r16] = O[nb][i];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) continue;
        sb[h * SW + HD] = mrun[h];
        sb[h * SW + HD + 1] = lrun[h];
      }
    }
    }
    if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
    mark(2);
    const int s_i = c->slen[P.i];
    const int c_first = cu_of(P.seg_start, W, nacu), c_last = cu_of(P.seg_start + s_i - 1, W, nacu);
    // CUs whose range is empty (fewer rows than CUs) hold no piece
    const int npieces = W >= nacu ? c_last - c_first + 1
                                   : (int)(cu_lo(c_last + 1, W, nacu) - cu_lo(c_first, W, nacu));
    float* ob = A->attn_out + ((size_t)l * A->bcap + P.i) * A->qdim + (size_t)P.g * G * HD;
    float* dst = apart_l + (size_t)(slot + P.sid) * pstride;
    // merge the four wave states: wave w takes heads w, w + 4; each lane HD/64 dims
    constexpr int DPL = HD / 64;
    const float* s0 = stb + (pidx & 1) * stride_st;
    for (int h = w; h < G; h += kComputeWaves) {
      float M = -INFINITY, L = 0.f, O[DPL];
#pragma unroll
      for (int k = 0; k < DPL; ++k) O[k] = 0.f;
#pragma unroll
      for (int ww = 0; ww < kComputeWaves; ++ww) {
        const float* e = s0 + ww * GM * SW + h * SW;
        const float m2 = e[HD], l2 = e[HD + 1];
        const float mn = fmaxf(M, m2);
        const float fa = mn == -INFINITY ? 0.f : exp2f(M - mn);
        const float fb = mn == -INFINITY ? 0.f : exp2f(m2 - mn);
#pragma unroll
        for (int k = 0; k < DPL; ++k) O[k] = O[k] * fa + e[DPL * lane + k] * fb;
        L = L * fa + l2 * fb;
        M = mn;
      }
      if (npieces == 1) {
        // the whole segment is here: normalise and store
        const float inv = 1.0f / L;
        const uint32_t tg = (tags >> P.i) & 1u;
        if constexpr (DPL == 2) co_store8(ob, (uint32_t)((h * HD + 2 * lane) * 4), u32x2{tagged(O[0] * inv, tg), tagged(O[1] * inv, tg)});
        else co_store_tag(ob, (uint32_t)((h * HD + lane) * 4), O[0] * inv, tg);
      } else {
        // every word with its lowest bit set: the finisher's validity flag
        if constexpr (DPL == 2) co_store8(dst, (uint32_t)((h * SW + 2 * lane) * 4), u32x2{tagged(O[0], 1u), tagged(O[1], 1u)});
        else co_store_tag(dst, (uint32_t)((h * SW + lane) * 4), O[0], 1u);
        if (lane == 0) co_store8(dst, (uint32_t)((h * SW + HD) * 4), u32x2{tagged(M, 1u), tagged(L, 1u)});
      }
    }
    mark(3);
    // a segment continued on other CUs is finished here once this CU's
    // pieces are done (only the last piece of a CU's range can be one)
    if (npieces > 1 && slot == c_first) {
      pend = Pend{P.sid, npieces, c_first, P.i, P.g, P.seg_start};
      has_pend = true;
    }
    mark(5);
    qc += P.nch;
    ++pidx;
    }
  }
  amark(1);
  if (has_pend) {
    if (!finish_segment(pend)) return false;
    mark(4);
  }
  amark(2);
  // the O projection polls the tagged outputs: no completion wait, no counter
  if (!cbar(A, c, s.gen, lane, &s.w_bar)) return false;
  s.synced = 1;
  mark(6);
#if MK_PHASE_TRACE
  if (ast) c->ppack = apack | ((uint64_t)(c->npoll & 0xFFFF) << 48);
  if (ast) c->npoll = 0;
#endif
  s.x_stage = -1;  // the staging buffer held softmax states
  return true;
}

template <int HD>
__device__ __forceinline__ bool attn_dispatch(DArgs A, TaskP tp, int cu, int w, int lane) {
  A = uni(A);
  if (A->G <= 1) return attn_task<HD, 1>(A, tp, cu, w, lane);
  if (A->G <= 2) return attn_task<HD, 2>(A, tp, cu, w, lane);
  if (A->G <= 4) return attn_task<HD, 4>(A, tp, cu, w, lane);
  if constexpr (HD == 64) return attn_task<HD, 8>(A, tp, cu, w, lane);
  return false;  // group > 4 at head_dim 128 is rejected at mk_create
}

__device__ __forceinline__ bool gemv_dispatch(DArgs A, TaskP tp, int cu, int w, int lane) {
  A = uni(A);
  if (A->mfma) return gemv_task<0>(A, tp, cu, w, lane);
  switch (A->b) {
    case 1: return gemv_task<1>(A, tp, cu, w, lane);
    case 2: return gemv_task<2>(A, tp, cu, w, lane);
    case 3: return gemv_task<3>(A, tp, cu, w, lane);
    case 4: return gemv_task<4>(A, tp, cu, w, lane);
    case 5: return gemv_task<5>(A, tp, cu, w, lane);
    case 6: return gemv_task<6>(A, tp, cu, w, lane);
    default: return gemv_task<7>(A, tp, cu, w, lane);
  }
}

__device__ __noinline__ void compute_main(DArgs A, int cu, int w, int lane) {
  A = uni(A);
  cu = __builtin_amdgcn_readfirstlane(cu);  // wave-uniform: scalar loads, no vmcnt drain
  w = __builtin_amdgcn_readfirstlane(w);
  Ctrl* c = ctrl_block(A);
  const TaskP T = as_const(A->tasks) + as_const(A->task_off)[cu];
  const int nt = as_const(A->task_off)[cu + 1] - as_const(A->task_off)[cu];
  CState& s = c->cs[w];
  s = CState{0, 0, 0, 0, 0, 0, 0, 0, -1, -1, -1, -1, -1, -1, -1, 1};
  const uint64_t t_kernel0 = A->trace ? now_ticks() : 0;
  uint64_t* tr = (A->trace && w == 0 && lane == 0) ? A->trace + (size_t)cu * A->trace_cap * 4 : nullptr;
  const int rpc = 4096 / A->hd;
  bool had_lm = false;
  for (int ti = 0; ti < nt; ++ti) {
    const Task t = load_task(uni(T + ti));
    const uint64_t t_begin = tr ? now_ticks() : 0;
    // no wait here: a task polls its tagged inputs itself (the schedule's
    // dependency counters order the streams and are checked on the host)
    const uint64_t t_dep = t_begin;
    s.t_stream = 0;
    bool ok;
    int nch = 0;
    if (t.type == TT_GEMV) {
      ok = gemv_dispatch(A, T + ti, cu, w, lane);
      nch = t.nchunks;
      had_lm = had_lm || t.stage == ST_LM;
    } else if (t.type == TT_ATTN) {
      ok = A->hd == 128 ? attn_dispatch<128>(A, T + ti, cu, w, lane) : attn_dispatch<64>(A, T + ti, cu, w, lane);
      nch = attn_task_chunks(A, cu, t.layer, rpc);
    } else if (t.type == TT_FIN) {
      ok = fin_task(A, T + ti, cu, w, lane);
      had_lm = had_lm || t.stage == ST_LM;
    } else {
      ok = embed_task(A, T + ti, cu, w, lane);
    }
    if (!ok) return;
    s.q += nch;
    if (tr && ti < A->trace_cap) {
      tr[ti * 4 + 0] = ((uint64_t)ti << 32) | ((uint64_t)(t.layer & 0xFFFF) << 16) | ((uint64_t)t.type << 8) | (uint64_t)t.stage;
      tr[ti * 4 + 1] = t_begin;
#if MK_PHASE_TRACE
      tr[ti * 4 + 2] = c->ppack;
      c->ppack = 0;
#else
      tr[ti * 4 + 2] = t_dep;
#endif
      tr[ti * 4 + 3] = now_ticks();
    }
  }
  if (A->trace && lane == 0) {
    uint64_t* st = A->trace + (size_t)A->ncu * A->trace_cap * 4 + (size_t)cu * kStatWords;
    st[4 + w] = s.w_empty;
    st[8 + w] = s.w_bar;
    st[16 + w] = s.t_math;
    st[20 + w] = s.t_stage;
    st[24 + w] = s.t_epi;
    if (w == 0) st[12] = now_ticks() - t_kernel0;
#if MK_PHASE_TRACE
    if (w == 0)
      for (int k = 0; k < 48; ++k) st[32 + k] = c->pstat[k];
#endif
  }
  // Greedy tokens: once every LM task has signalled, the argmax keys are
  // final.  Every CU that ran LM tasks checks once; the CU whose signal was
  // the last one is guaranteed to see completion (duplicates write the same
  // values).
  if (w == 0 && had_lm && A->next_tokens) {
    wait_mem();
    const int ctr = ctr_lm(A->L);
    const uint32_t* p = bank_ptr(A, A->bank) + lane * A->ctr_stride + ctr;
    int v = (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(v >= as_const(A->expect)[ctr * kShards + lane]) && lane < A->b) {
      unsigned long long key = __hip_atomic_load(keys_ptr(A) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      A->next_tokens[lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void mk_step_kernel(DevArgs args) {
  (void)args;
  DArgs A = (DArgs)__builtin_amdgcn_kernarg_segment_ptr();
  Ctrl* c = ctrl_block(A);
#ifndef MK_XCD_MAP
#define MK_XCD_MAP 0
#endif
  // MK_XCD_MAP: work-groups are dealt round-robin over the 8 XCDs, so plan
  // CU p = (block % 8) * (grid / 8) + block / 8 puts consecutive plan CUs on
  // one XCD (and its L2)
  const int cu = (MK_XCD_MAP && gridDim.x % 8 == 0) ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                                                    : (int)blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  // zero this CU's slice of the bank the next step will use
  {
    uint32_t* nb = bank_ptr(A, A->bank ^ 1);
    const int per = (A->bank_words + A->ncu - 1) / A->ncu;
    const int lo = cu * per, hi = min(A->bank_words, lo + per);
    for (int i = lo + tid; i < hi; i += kThreads) nb[i] = 0u;
  }
  if (tid < kMaxSlots) {
    c->ready[tid] = 0;
    c->freed[tid] = 0;
  }
  if (tid < kMaxBatch) c->lmkey[tid] = 0ull;
#if MK_PHASE_TRACE
  if (tid < 48) c->pstat[tid] = 0;
  if (tid == 0) {
    c->ppack = 0;
    c->npoll = 0;
  }
#endif
  if (tid == 0) {
    c->dep = 0;
    c->bar = 0;
    c->fin = 0;
    c->abort = 0;
  }
  // per-sequence inputs, validated and clamped identically on every CU
  if (tid < A->b) {
    uint32_t st = 0;
    int tok = A->tokens[tid];
    if (tok < 0 || tok >= A->V) {
      st |= 1u;
      tok = tok < 0 ? 0 : A->V - 1;
    }
    int p = A->positions[tid];
    const int cap = min(A->max_seq, A->kv_scap);
    if (p < 0 || p >= cap) {
      st |= 2u;
      p = p < 0 ? 0 : cap - 1;
    }
    if (A->seq_lens[tid] != A->positions[tid] + 1) st |= 4u;
    c->tok[tid] = tok;
    c->pos[tid] = p;
    c->slen[tid] = p + 1;
    if (st && cu == 0) atomicOr(A->status, st);
  }
  __syncthreads();
  if (w < kComputeWaves) compute_main(A, cu, w, lane);
  else loader_main(A, cu, w - kComputeWaves, lane);
}

size_t lds_bytes(int nslot, int xb_bytes) {
  return (size_t)nslot * kSlotBytes + xb_bytes + kRedBytes + kCtrlBytes;
}

static hipError_t set_lds_limit(size_t lds) {
  static size_t lds_set = 0;
  if (lds > lds_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mk_step_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set = lds;
  }
  return hipSuccess;
}

// Work-groups of the step kernel that fit one CU at the given dynamic LDS
// size (0 when they do not fit at all).
hipError_t step_occupancy(size_t lds, int* blocks_per_cu) {
  hipError_t e = set_lds_limit(lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)mk_step_kernel, kThreads, lds);
}

// One launch of ncu persistent work-groups.  The work-groups poll each other,
// so all of them must be resident at once: a cooperative launch has the
// runtime guarantee that (it fails rather than start a partial grid).
hipError_t launch_step(const DevArgs& A, hipStream_t stream, bool coop) {
  const size_t lds = lds_bytes(A.nslot, A.xb_bytes);
  hipError_t e = set_lds_limit(lds);
  if (e != hipSuccess) return e;
  if (coop) {
    void* args[] = {(void*)&A};
    return hipLaunchCooperativeKernel((const void*)mk_step_kernel, dim3(A.ncu), dim3(kThreads), args, (unsigned)lds,
                                      stream);
  }
  hipLaunchKernelGGL(mk_step_kernel, dim3(A.ncu), dim3(kThreads), lds, stream, A);
  return hipGetLastError();
}

// ---- scratch of the allocation-free step: a file-scope device array.  Host
// code never uses the array's name as an address: its device address is
// looked up once per device (with that device current) and kept.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch_base(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* base[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    base[dev] = p;
  }
  *out = base[dev];
  return hipSuccess;
}

// Zero `bytes` (a multiple of 16) at p: a kernel rather than a memset node, so
// a caller may capture the call into a graph.
__global__ void mk_zero_kernel(u32x4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  hipLaunchKernelGGL(mk_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4*)p, n);
  return hipGetLastError();
}

// Copy of `rows` rows of 32-bit activation words with the step-tag bit
// cleared (pitches and row length in bytes, multiples of 4).
__global__ void mk_untag_copy_kernel(uint32_t* dst, size_t dpitch, const uint32_t* src, size_t spitch, size_t words,
                                     size_t rows) {
  const size_t total = words * rows;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / words, k = i - r * words;
    dst[r * dpitch + k] = src[r * spitch + k] & ~1u;
  }
}

hipError_t launch_untag_copy(void* dst, size_t dpitch, const void* src, size_t spitch, size_t row_bytes, size_t rows,
                             hipStream_t stream) {
  const size_t words = row_bytes / 4, total = words * rows;
  if (total == 0) return hipSuccess;
  const size_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(mk_untag_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)dst, dpitch / 4,
                     (const uint32_t*)src, spitch / 4, words, rows);
  return hipGetLastError();
}

}  // namespace mk
