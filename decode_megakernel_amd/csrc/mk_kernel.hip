// Persistent decode-step megakernel for gfx950 (MI355X).
//
// One work-group per CU walks that CU's instruction stream (built on the host,
// see mk_plan.cpp).  Inside a work-group:
//   * 4 loader waves stream every input-independent byte the CU's tasks need
//     (weight tiles, cached K/V rows) from HBM into an LDS ring with
//     non-temporal loads.  They never wait on a dependency counter, so weights
//     for later tasks arrive while the CU is still waiting for activations
//     (the weight prefetch of the Cohere megakernel digest; the shared-memory
//     buffer pool of the ForgeMegakernel milestones).
//   * 4 compute waves wait on dependency counters, stage the activation slice
//     into LDS, run the GEMV (VALU dot2 for small batches, MFMA 16x16x32 bf16
//     for batch >= 8) or split-KV attention tiles out of the ring, and write
//     their outputs with fused epilogues (residual add, next RMSNorm's sum of
//     squares, SiLU-gate, RoPE, KV store, argmax).
// Cross-CU exchange uses device-coherent (sc1) loads and stores plus 64-way
// sharded counters; no agent-scope cache fences are issued on the hot path.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr unsigned kCpSc1 = 16;  // cache policy: device scope (coherent across XCDs)
constexpr uint32_t kStatusTimeout = 8u;

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7FFFFFFF, 0x00020000);
}
// device-coherent accesses; byte offsets relative to a wave-uniform base
__device__ __forceinline__ u32x4 co_load16(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, kCpSc1);
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

// LDS accessors
__device__ __forceinline__ u32x4 lds_ld16(const char* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void lds_st16(char* p, u32x4 v) { *(u32x4*)p = v; }

// ------------------------------------------------------------ CU control
struct Ctrl {
  int ready[kMaxSlots];
  int freed[kMaxSlots];
  int dep;
  int bar;
  int fin;
  int abort;
  int pos[kMaxBatch];
  int slen[kMaxBatch];
  int tok[kMaxBatch];
  float rms[kMaxBatch];
};

__device__ __forceinline__ int lds_ld_acq(int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ void lds_st_rel(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ bool lds_aborted(Ctrl* c) { return __hip_atomic_load(&c->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0; }

__device__ __forceinline__ bool global_aborted(const DevArgs& A) {
  return __hip_atomic_load(A.status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Every spin loop is bounded: on abort or after the time limit the CU gives
// up (the time limit also raises MK_STATUS_TIMEOUT), so the kernel always
// terminates.
struct Spin {
  uint64_t t0;
  int it;
};
__device__ __forceinline__ Spin spin_start() { return Spin{now_ticks(), 0}; }
__device__ __noinline__ bool spin_fail(const DevArgs& A, Ctrl* c) {
  if (__hip_atomic_load(&c->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return true;
  if (global_aborted(A)) {
    __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
  }
  return false;
}
// returns false when the wait must be abandoned
__device__ __forceinline__ bool spin_ok(const DevArgs& A, Ctrl* c, Spin& sp) {
  if (lds_aborted(c)) return false;
  if ((++sp.it & 63) == 0) {
    if (spin_fail(A, c)) return false;
    if (now_ticks() - sp.t0 > A.timeout_ticks) {
      atomicOr(A.status, kStatusTimeout);
      __hip_atomic_store(A.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

// Software barrier among the compute waves (the loader waves never join).
__device__ __forceinline__ bool cbar(const DevArgs& A, Ctrl* c, int& gen, int lane) {
  ++gen;
  if (lane == 0) __hip_atomic_fetch_add(&c->bar, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int target = gen * kComputeWaves;
  Spin sp = spin_start();
  while (lds_ld_acq(&c->bar) < target)
    if (!spin_ok(A, c, sp)) return false;
  return true;
}

__device__ __forceinline__ uint32_t* bank_ptr(const DevArgs& A, int which) {
  return A.banks + (size_t)which * A.bank_words;
}
__device__ __forceinline__ unsigned long long* keys_ptr(const DevArgs& A) {
  return (unsigned long long*)(bank_ptr(A, A.bank) + kShards * A.ctr_stride);
}

// Wait (one wave, all 64 lanes) until every shard of counter `ctr` reached
// the count the schedule expects.
__device__ bool wait_counter(const DevArgs& A, Ctrl* c, int ctr, int lane) {
  const uint32_t* p = bank_ptr(A, A.bank) + lane * A.ctr_stride + ctr;
  const int e = A.expect[ctr * kShards + lane];
  const uint64_t t0 = now_ticks();
  for (int it = 0;; ++it) {
    int v = (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(v >= e)) return true;
    if ((it & 15) == 15) {
      if (global_aborted(A)) {
        __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return false;
      }
      if (now_ticks() - t0 > A.timeout_ticks) {
        if (lane == 0) {
          atomicOr(A.status, kStatusTimeout);
          __hip_atomic_store(A.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(&c->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ void signal_counter(const DevArgs& A, int ctr, int cu) {
  uint32_t* p = bank_ptr(A, A.bank) + (cu % kShards) * A.ctr_stride + ctr;
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------- stage geometry
__device__ __forceinline__ int stage_M(const DevArgs& A, int st) {
  switch (st) {
    case ST_QKV: return A.nqkv;
    case ST_O: return A.d;
    case ST_GU: return 2 * A.I;
    case ST_DOWN: return A.d;
    default: return A.V;
  }
}
__device__ __forceinline__ int stage_K(const DevArgs& A, int st) {
  switch (st) {
    case ST_O: return A.qdim;
    case ST_DOWN: return A.I;
    default: return A.d;
  }
}
// bf16 input activation [bcap][K] of a GEMV stage
__device__ __forceinline__ const uint16_t* stage_x(const DevArgs& A, int st, int l) {
  switch (st) {
    case ST_QKV: return A.xattn + (size_t)l * A.bcap * A.d;
    case ST_O: return A.attn_out + (size_t)l * A.bcap * A.qdim;
    case ST_GU: return A.xmlp + (size_t)l * A.bcap * A.d;
    case ST_DOWN: return A.act + (size_t)l * A.bcap * A.I;
    default: return A.xattn + (size_t)A.L * A.bcap * A.d;  // LM head reads the final-normed input
  }
}
__device__ __forceinline__ const float* stage_ss(const DevArgs& A, int st, int l) {
  const int nt = A.d / 16;
  switch (st) {
    case ST_QKV: return A.ssattn + (size_t)l * nt * A.bcap;
    case ST_GU: return A.ssmlp + (size_t)l * nt * A.bcap;
    case ST_LM: return A.ssattn + (size_t)A.L * nt * A.bcap;
    default: return nullptr;
  }
}
// weight row `lr` (logical row of the stage) of layer l
__device__ __forceinline__ const uint16_t* row_ptr(const DevArgs& A, int st, int l, int lr) {
  switch (st) {
    case ST_QKV: {
      const LayerW& w = A.layers[l];
      if (lr < A.qdim) return w.q + (size_t)lr * A.d;
      lr -= A.qdim;
      if (lr < A.kvdim) return w.k + (size_t)lr * A.d;
      return w.v + (size_t)(lr - A.kvdim) * A.d;
    }
    case ST_O: return A.layers[l].o + (size_t)lr * A.qdim;
    case ST_GU: {
      // logical tile t = 8 gate rows (8t..8t+7) followed by the same 8 up rows
      const LayerW& w = A.layers[l];
      int t = lr >> 4, j = lr & 15;
      return (j < 8 ? w.gate : w.up) + (size_t)(8 * t + (j & 7)) * A.d;
    }
    case ST_DOWN: return A.layers[l].down + (size_t)lr * A.I;
    default: return A.lm_head + (size_t)lr * A.d;
  }
}

// ---------------------------------------------------- attention partition
// The flattened attention work of a step is the (sequence, kv-head, position)
// rows in that order; CU c owns rows [W*c/ncu, W*(c+1)/ncu).  Every CU derives
// the same partition from seq_lens, so a ragged batch is balanced without a
// host round trip and without broadcasting one sequence's position.
struct Piece {
  int i, g, j0, j1, sid, ncached, nch, has_new;
  long long seg_start;
};

__device__ __forceinline__ long long attn_total(const Ctrl* c, int b, int nkv) {
  long long W = 0;
  for (int i = 0; i < b; ++i) W += c->slen[i];
  return W * nkv;
}
__device__ __forceinline__ long long cu_lo(int cu, long long W, int ncu) { return W * cu / ncu; }
__device__ __forceinline__ int cu_of(long long x, long long W, int ncu) {
  return (int)(((x + 1) * ncu + W - 1) / W) - 1;
}

__device__ __forceinline__ bool next_piece(const Ctrl* c, int b, int nkv, int rpc, long long& pos, long long hi, Piece& P) {
  if (pos >= hi) return false;
  long long acc = 0;
  int i = 0;
  for (; i < b - 1; ++i) {
    long long seg = (long long)nkv * c->slen[i];
    if (pos < acc + seg) break;
    acc += seg;
  }
  const int s = c->slen[i];
  long long off = pos - acc;
  P.i = i;
  P.g = (int)(off / s);
  P.j0 = (int)(off % s);
  long long take = s - P.j0;
  if (hi - pos < take) take = hi - pos;
  P.j1 = P.j0 + (int)take;
  P.sid = i * nkv + P.g;
  P.seg_start = acc + (long long)P.g * s;
  const int p = s - 1;
  int nc = (P.j1 < p ? P.j1 : p) - P.j0;
  P.ncached = nc > 0 ? nc : 0;
  P.has_new = P.j1 == s;
  P.nch = (P.ncached + rpc - 1) / rpc;
  pos += take;
  return true;
}

// ================================================================ loader
struct LDesc {
  int task;     // index into this CU's stream
  int local;    // chunk index within the task
  int q;        // CU-global chunk sequence number
};

struct LoaderIter {
  int ti, nt, qbase, nchunks, entered, q;
};

__device__ int attn_task_chunks(const DevArgs& A, const Ctrl* c, int cu, int rpc) {
  long long W = attn_total(c, A.b, A.nkv);
  long long pos = cu_lo(cu, W, A.ncu), hi = cu_lo(cu + 1, W, A.ncu);
  Piece P;
  int n = 0;
  while (next_piece(c, A.b, A.nkv, rpc, pos, hi, P)) n += P.nch;
  return n;
}

__device__ bool loader_next(const DevArgs& A, const Task* T, const Ctrl* c, int cu, int rpc, LoaderIter& it, LDesc& d) {
  while (it.ti < it.nt) {
    if (!it.entered) {
      const Task& t = T[it.ti];
      if (t.type == TT_GEMV) it.nchunks = t.nchunks;
      else if (t.type == TT_ATTN) it.nchunks = attn_task_chunks(A, c, cu, rpc);
      else it.nchunks = 0;
      it.entered = 1;
    }
    if (it.q < it.qbase + it.nchunks) {
      d.task = it.ti;
      d.local = it.q - it.qbase;
      d.q = it.q;
      it.q += kLoaderWaves;
      return true;
    }
    it.qbase += it.nchunks;
    it.ti += 1;
    it.entered = 0;
  }
  return false;
}

template <int HD>
__device__ __forceinline__ void issue_attn_loads(const DevArgs& A, const Ctrl* c, const Task& t, int cu, int local, int lane, u32x4* r) {
  constexpr int LPR = HD / 8, RP = 64 / LPR, RPC = 4096 / HD;
  long long W = attn_total(c, A.b, A.nkv);
  long long pos = cu_lo(cu, W, A.ncu), hi = cu_lo(cu + 1, W, A.ncu);
  Piece P;
  int base = 0;
  while (next_piece(c, A.b, A.nkv, RPC, pos, hi, P)) {
    if (local < base + P.nch) break;
    base += P.nch;
  }
  const int ch = local - base;
  const int rows = min(RPC, P.ncached - ch * RPC);
  const size_t head = (((size_t)t.layer * A.kv_bcap + P.i) * A.nkv + P.g) * A.kv_scap;
  const int e = (lane % LPR) * 8;
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) {
    const int rl = (j & 7) * RP + lane / LPR;
    const uint16_t* src = (j < 8 ? A.kc : A.vc) + (head + P.j0 + ch * RPC + rl) * HD + e;
    r[j] = rl < rows ? nt_load16(src) : u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void issue_gemv_loads(const DevArgs& A, const Task& t, int local, int lane, u32x4* r) {
  const int M = stage_M(A, t.stage);
  if (!A.mfma) {
    const int kk = t.k0 + kValuBlock * local + 8 * lane;
#pragma unroll
    for (int j = 0; j < kWaveLoads; ++j) {
      const int lr = t.row0 + j;
      const bool ok = lr < M && kk < t.k1;
      r[j] = ok ? nt_load16(row_ptr(A, t.stage, t.layer, lr) + kk) : u32x4{0, 0, 0, 0};
    }
  } else {
    const int R = t.nsub, spc = kWaveLoads / R;
#pragma unroll
    for (int j = 0; j < kWaveLoads; ++j) {
      const int s = j / R, rr = j % R;
      const int kk = t.k0 + 32 * (local * spc + s) + 8 * (lane >> 4);
      const int lr = t.row0 + 16 * rr + (lane & 15);
      const bool ok = lr < M && kk < t.k1;
      r[j] = ok ? nt_load16(row_ptr(A, t.stage, t.layer, lr) + kk) : u32x4{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ void issue_loads(const DevArgs& A, const Task* T, const Ctrl* c, int cu, const LDesc& d, int lane, u32x4* r) {
  const Task& t = T[d.task];
  if (t.type == TT_GEMV) issue_gemv_loads(A, t, d.local, lane, r);
  else if (A.hd == 128) issue_attn_loads<128>(A, c, t, cu, d.local, lane, r);
  else issue_attn_loads<64>(A, c, t, cu, d.local, lane, r);
}

__device__ __forceinline__ bool store_chunk(const DevArgs& A, char* ring, Ctrl* c, const LDesc& d, int lane, const u32x4* r) {
  const int slot = d.q % A.nslot;
  const int need = d.q - A.nslot + 1;
  Spin sp = spin_start();
  while (lds_ld_acq(&c->freed[slot]) < need)
    if (!spin_ok(A, c, sp)) return false;
  char* dst = ring + (size_t)slot * kChunkBytes + lane * 16;
#pragma unroll
  for (int j = 0; j < kWaveLoads; ++j) lds_st16(dst + j * 1024, r[j]);
  if (lane == 0) lds_st_rel(&c->ready[slot], d.q + 1);
  return true;
}

__device__ void loader_main(const DevArgs& A, char* ring, Ctrl* c, int cu, int lw, int lane) {
  const Task* T = A.tasks + A.task_off[cu];
  const int rpc = 4096 / A.hd;
  LoaderIter it{0, A.task_off[cu + 1] - A.task_off[cu], 0, 0, 0, lw};
  LDesc da, db;
  u32x4 ra[kWaveLoads], rb[kWaveLoads];
  bool have_a = loader_next(A, T, c, cu, rpc, it, da);
  if (have_a) issue_loads(A, T, c, cu, da, lane, ra);
  while (have_a) {
    bool have_b = loader_next(A, T, c, cu, rpc, it, db);
    if (have_b) issue_loads(A, T, c, cu, db, lane, rb);
    if (!store_chunk(A, ring, c, da, lane, ra)) return;
    if (!have_b) break;
    have_a = loader_next(A, T, c, cu, rpc, it, da);
    if (have_a) issue_loads(A, T, c, cu, da, lane, ra);
    if (!store_chunk(A, ring, c, db, lane, rb)) return;
  }
}

// ================================================================ compute
struct CState {
  int gen;      // compute-barrier generation
  int q;        // chunk sequence number of the current task's first chunk
  int last_dep; // counter of the last dependency already satisfied
  int x_stage, x_layer, x_k0, x_k1;  // signature of the staged input slice
};

__device__ __forceinline__ bool wait_chunk(const DevArgs& A, Ctrl* c, int gq) {
  const int slot = gq % A.nslot;
  Spin sp = spin_start();
  while (lds_ld_acq(&c->ready[slot]) < gq + 1)
    if (!spin_ok(A, c, sp)) return false;
  return true;
}
__device__ __forceinline__ void free_chunk(const DevArgs& A, Ctrl* c, int gq, int lane) {
  if (lane == 0) lds_st_rel(&c->freed[gq % A.nslot], gq + 1);
}

// Wave-wide sum over 16-lane groups (lanes l, l^1, ..., l^8).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// Order-preserving 64-bit key: larger logit first, then lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  v = v + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (uint32_t)idx);
}

// ---- stage the GEMV input slice x[n][k0:k1] (bf16) into LDS, and the RMS
//      scales of the stages that normalize their input.
__device__ bool stage_input(const DevArgs& A, const Task& t, char* xb, Ctrl* c, CState& s, int w, int lane) {
  if (s.x_stage == t.stage && s.x_layer == t.layer && s.x_k0 == t.k0 && s.x_k1 == t.k1) return true;
  const int K = stage_K(A, t.stage);
  const int ksl = t.k1 - t.k0, ksp = ksl + 8;
  const uint16_t* x = stage_x(A, t.stage, t.layer);
  const int per_row = ksl / 8;
  const int units = A.b * per_row;
  const int tid = w * 64 + lane;
  for (int u = tid; u < units; u += kComputeThreads) {
    int n = u / per_row, kq = u - n * per_row;
    u32x4 v = co_load16(x, (uint32_t)(((size_t)n * K + t.k0 + 8 * kq) * 2));
    lds_st16(xb + ((size_t)n * ksp + 8 * kq) * 2, v);
  }
  const float* ss = stage_ss(A, t.stage, t.layer);
  if (ss) {
    const int nt = A.d / 16;
    for (int n = w; n < A.b; n += kComputeWaves) {
      float acc = 0.f;
      for (int i = lane; i < nt; i += 64) acc += co_loadf(ss, (uint32_t)(((size_t)i * A.bcap + n) * 4));
      for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
      if (lane == 0) c->rms[n] = 1.0f / sqrtf(acc / (float)A.d + A.eps);
    }
  }
  s.x_stage = t.stage;
  s.x_layer = t.layer;
  s.x_k0 = t.k0;
  s.x_k1 = t.k1;
  return cbar(A, c, s.gen, lane);
}

// ---- VALU chunk: 16 rows x 512 K; lane l covers K elements [8l, 8l+8)
template <int NB>
__device__ __forceinline__ void valu_chunk(const char* slot, const char* xb, int ksp, int kl, int lane, float (&acc)[16][NB]) {
  u32x4 xv[NB];
  const bool ok = kl < ksp - 8;  // inside the slice (ksp = slice + 8)
#pragma unroll
  for (int n = 0; n < NB; ++n) xv[n] = ok ? lds_ld16(xb + ((size_t)n * ksp + kl) * 2) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    u32x4 wv = lds_ld16(slot + j * 1024 + lane * 16);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[j][n] = dot8_bf16(wv, xv[n], acc[j][n]);
  }
}

// Reduce acc[16][NB] over the 64 lanes with a transposing butterfly; lane l
// ends with the total of row ((l>>5)&1)*8 + ((l>>4)&1)*4 + ((l>>3)&1)*2 + ((l>>2)&1).
template <int NB>
__device__ __forceinline__ void valu_reduce(float (&acc)[16][NB], int lane, float* out /*[NB]*/) {
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    float v8[8], v4[4], v2[2], v1;
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float send = b5 ? acc[r][n] : acc[r + 8][n];
      float keep = b5 ? acc[r + 8][n] : acc[r][n];
      v8[r] = keep + __shfl_xor(send, 32);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float send = b4 ? v8[r] : v8[r + 4];
      float keep = b4 ? v8[r + 4] : v8[r];
      v4[r] = keep + __shfl_xor(send, 16);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float send = b3 ? v4[r] : v4[r + 2];
      float keep = b3 ? v4[r + 2] : v4[r];
      v2[r] = keep + __shfl_xor(send, 8);
    }
    {
      float send = b2 ? v2[0] : v2[1];
      float keep = b2 ? v2[1] : v2[0];
      v1 = keep + __shfl_xor(send, 4);
    }
    v1 += __shfl_xor(v1, 2);
    v1 += __shfl_xor(v1, 1);
    out[n] = v1;
  }
}

// ---- MFMA chunk: R sub-tiles x (16/R) k-steps of 32
template <int R>
__device__ __forceinline__ void mfma_chunk(const char* slot, const char* xb, int ksp, int kstep0, int nsteps, int b, int lane, f32x4 (&acc)[R]) {
  constexpr int SPC = kWaveLoads / R;
  const int n = lane & 15, kq = 8 * (lane >> 4);
#pragma unroll
  for (int s = 0; s < SPC; ++s) {
    if (kstep0 + s >= nsteps) break;
    const int kl = 32 * (kstep0 + s) + kq;
    u32x4 bv = n < b ? lds_ld16(xb + ((size_t)n * ksp + kl) * 2) : u32x4{0, 0, 0, 0};
    bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bv);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      u32x4 av = lds_ld16(slot + (s * R + r) * 1024 + lane * 16);
      acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), bb, acc[r], 0, 0, 0);
    }
  }
}

// Epilogue of one output element (row `lr` of the stage, sequence n) of a
// complete tile.  Threads map t -> (n = t >> 4, row = t & 15), so each
// 16-lane group holds one sequence's 16 consecutive rows.
__device__ void gemv_epilogue(const DevArgs& A, const Task& t, Ctrl* c, int r, int row, int n, float val, float val_up, int lane) {
  const int l = t.layer;
  const int M = stage_M(A, t.stage);
  const int lr = t.row0 + 16 * r + row;
  const bool valid = n < A.b && lr < M;
  switch (t.stage) {
    case ST_QKV:
      if (valid) co_storef(A.qkv, (uint32_t)((((size_t)l * A.bcap + n) * A.nqkv + lr) * 4), c->rms[n] * val);
      break;
    case ST_O:
    case ST_DOWN: {
      // h = residual + projection; also the next RMSNorm's input and its
      // per-16-row sum of squares.
      const bool down = t.stage == ST_DOWN;
      const float* hin = down ? A.hmid + (size_t)l * A.bcap * A.d : A.hres + (size_t)l * A.bcap * A.d;
      float* hout = down ? A.hres + (size_t)(l + 1) * A.bcap * A.d : A.hmid + (size_t)l * A.bcap * A.d;
      uint16_t* xo = down ? A.xattn + (size_t)(l + 1) * A.bcap * A.d : A.xmlp + (size_t)l * A.bcap * A.d;
      const uint16_t* nw = down ? (l + 1 < A.L ? A.layers[l + 1].attn_norm : A.final_norm) : A.layers[l].mlp_norm;
      float* ssout = down ? A.ssattn + (size_t)(l + 1) * (A.d / 16) * A.bcap : A.ssmlp + (size_t)l * (A.d / 16) * A.bcap;
      const uint32_t off = (uint32_t)(((size_t)n * A.d + lr) * 4);
      float h = valid ? co_loadf(hin, off) + val : 0.f;
      float xn = valid ? h * bf2f(nw[lr]) : 0.f;
      float xn_next = __shfl_down(xn, 1);
      if (valid) {
        co_storef(hout, off, h);
        if ((row & 1) == 0) co_store4(xo, (uint32_t)(((size_t)n * A.d + lr) * 2), pack_bf2(xn, xn_next));
      }
      float ss = sum16(h * h);
      if (valid && row == 0) co_storef(ssout, (uint32_t)((((size_t)lr >> 4) * A.bcap + n) * 4), ss);
      break;
    }
    case ST_GU: {
      // rows 0-7 of a 16-row logical tile are gate rows, 8-15 the same up rows
      float a = 0.f;
      if (valid && row < 8) {
        float g = c->rms[n] * val, u = c->rms[n] * val_up;
        a = g / (1.0f + __expf(-g)) * u;
      }
      float a_next = __shfl_down(a, 1);
      if (valid && row < 8 && (row & 1) == 0) {
        const int out = 8 * ((t.row0 >> 4) + r) + row;
        co_store4(A.act, (uint32_t)((((size_t)l * A.bcap + n) * A.I + out) * 2), pack_bf2(a, a_next));
      }
      break;
    }
    default: {  // LM head + greedy argmax
      float v = valid ? c->rms[n] * val : 0.f;
      if (valid) A.logits[(size_t)n * A.V + lr] = v;
      unsigned long long key = valid ? argmax_key(v, lr) : 0ull;
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        unsigned long long o = ((unsigned long long)(uint32_t)__shfl_xor((int)(key >> 32), m) << 32) |
                               (uint32_t)__shfl_xor((int)(uint32_t)key, m);
        key = o > key ? o : key;
      }
      if (row == 0 && n < A.b && key) __hip_atomic_fetch_max(keys_ptr(A) + n, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

template <int NB, int R>
__device__ bool gemv_task(const DevArgs& A, const Task& t, char* ring, char* xb, float* red, Ctrl* c, CState& s, int cu, int w, int lane) {
  if (!stage_input(A, t, xb, c, s, w, lane)) return false;
  const int ksp = (t.k1 - t.k0) + 8;
  // ---- stream the task's chunks (chunk q belongs to compute wave q % 4)
  float vacc[16][NB];
  f32x4 macc[R];
  if (!A.mfma) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int n = 0; n < NB; ++n) vacc[j][n] = 0.f;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) macc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nsteps = (t.k1 - t.k0) / 32;
  for (int local = 0; local < t.nchunks; ++local) {
    const int gq = s.q + local;
    if ((gq & (kComputeWaves - 1)) != w) continue;
    if (!wait_chunk(A, c, gq)) return false;
    const char* slot = ring + (size_t)(gq % A.nslot) * kChunkBytes;
    if (!A.mfma) valu_chunk<NB>(slot, xb, ksp, kValuBlock * local + 8 * lane, lane, vacc);
    else mfma_chunk<R>(slot, xb, ksp, local * (kWaveLoads / R), nsteps, A.b, lane, macc);
    free_chunk(A, c, gq, lane);
  }
  // ---- per-wave partial sums -> LDS
  float* rw = red + w * 1024;
  if (!A.mfma) {
    float tot[NB];
    valu_reduce<NB>(vacc, lane, tot);
    if ((lane & 3) == 0) {
      const int row = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
#pragma unroll
      for (int n = 0; n < NB; ++n) rw[row * 16 + n] = tot[n];
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) *(f32x4*)(rw + (r * 64 + lane) * 4) = macc[r];
  }
  if (!cbar(A, c, s.gen, lane)) return false;
  // ---- combine the 4 waves; thread -> (n, row)
  const int tid = w * 64 + lane, n = tid >> 4, row = tid & 15;
  auto value = [&](int r, int rw_) -> float {
    float v = 0.f;
    if (!A.mfma) {
#pragma unroll
      for (int ww = 0; ww < kComputeWaves; ++ww) v += red[ww * 1024 + rw_ * 16 + n];
    } else {
      const int src = n + 16 * (rw_ >> 2), i = rw_ & 3;
#pragma unroll
      for (int ww = 0; ww < kComputeWaves; ++ww) v += red[ww * 1024 + (r * 64 + src) * 4 + i];
    }
    return v;
  };
  const int Rn = A.mfma ? R : 1;
  float vals[R], ups[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    vals[r] = r < Rn ? value(r, row) : 0.f;
    ups[r] = (r < Rn && t.stage == ST_GU && row < 8) ? value(r, row + 8) : 0.f;
  }
  if (t.nks > 1) {
    // split-K: publish this slice's partial; the last slice of the group sums
    // all partials in slice order and runs the epilogue.
    float* pb = A.part + (size_t)(t.part_slot + t.ks) * 1024;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < Rn) co_storef(pb, (uint32_t)((r * 256 + tid) * 4), vals[r]);
    wait_mem();
    if (!cbar(A, c, s.gen, lane)) return false;
    if (w == 0) {
      int fin = 0;
      if (lane == 0) {
        uint32_t* gc = A.grp_ctr + A.grp_off[t.stage] + t.group;
        uint32_t old = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        fin = (int)old == t.nks - 1;
        if (fin) __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_st_rel(&c->fin, fin);
      }
    }
    if (!cbar(A, c, s.gen, lane)) return false;
    if (lds_ld_acq(&c->fin)) {
      const float* p0 = A.part + (size_t)t.part_slot * 1024;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= Rn) continue;
        float v = 0.f, u = 0.f;
        for (int k = 0; k < t.nks; ++k) {
          v += co_loadf(p0, (uint32_t)(((size_t)k * 1024 + r * 256 + tid) * 4));
          if (t.stage == ST_GU && row < 8) u += co_loadf(p0, (uint32_t)(((size_t)k * 1024 + r * 256 + tid + 8) * 4));
        }
        vals[r] = v;
        ups[r] = u;
      }
    } else {
      wait_mem();
      if (!cbar(A, c, s.gen, lane)) return false;
      if (w == 0 && lane == 0) signal_counter(A, t.signal_ctr, cu);
      return true;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < Rn) gemv_epilogue(A, t, c, r, row, n, vals[r], ups[r], lane);
  wait_mem();
  if (!cbar(A, c, s.gen, lane)) return false;
  if (w == 0 && lane == 0) signal_counter(A, t.signal_ctr, cu);
  return true;
}

// ---- embedding gather: h0 = E[token] for 64 columns, plus the first
//      RMSNorm's input and per-16-column sums of squares.
__device__ bool embed_task(const DevArgs& A, const Task& t, Ctrl* c, CState& s, int cu, int w, int lane) {
  const int tid = w * 64 + lane, n = tid >> 4, col = t.row0 + 4 * (tid & 15);
  float h[4] = {0.f, 0.f, 0.f, 0.f};
  const bool valid = n < A.b;
  if (valid) {
    const uint16_t* e = A.embed + (size_t)c->tok[n] * A.d + col;
    u32x2 ev = *(const u32x2*)e;
    h[0] = bf_lo(ev.x); h[1] = bf_hi(ev.x); h[2] = bf_lo(ev.y); h[3] = bf_hi(ev.y);
    const uint16_t* nw = A.layers[0].attn_norm + col;
    co_store16(A.hres, (uint32_t)(((size_t)n * A.d + col) * 4),
               u32x4{__float_as_uint(h[0]), __float_as_uint(h[1]), __float_as_uint(h[2]), __float_as_uint(h[3])});
    co_store8(A.xattn, (uint32_t)(((size_t)n * A.d + col) * 2),
              u32x2{pack_bf2(h[0] * bf2f(nw[0]), h[1] * bf2f(nw[1])), pack_bf2(h[2] * bf2f(nw[2]), h[3] * bf2f(nw[3]))});
  }
  float ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  if (valid && (tid & 3) == 0) co_storef(A.ssattn, (uint32_t)((((size_t)col >> 4) * A.bcap + n) * 4), ss);
  wait_mem();
  if (!cbar(A, c, s.gen, lane)) return false;
  if (w == 0 && lane == 0) signal_counter(A, t.signal_ctr, cu);
  return true;
}

// ---- attention --------------------------------------------------------
struct SoftState {
  float m, l;
};

// Load a head's 8 own elements and the 8 rotate-half partners of a raw q/k
// row (fp32 in the qkv buffer), apply the optional per-head RMSNorm and RoPE.
template <int HD>
__device__ __forceinline__ void rope_head(const DevArgs& A, const float* src /* head base */, const uint16_t* normw, int p, int e0, float* out) {
  constexpr int LPR = HD / 8;
  u32x4 a0 = co_load16(src, (uint32_t)(e0 * 4)), a1 = co_load16(src, (uint32_t)((e0 + 4) * 4));
  const int pe = (e0 + HD / 2) % HD;
  u32x4 b0 = co_load16(src, (uint32_t)(pe * 4)), b1 = co_load16(src, (uint32_t)((pe + 4) * 4));
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
    const float rs = 1.0f / sqrtf(ss / (float)HD + A.eps);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      x[u] = x[u] * rs * bf2f(normw[e0 + u]);
      y[u] = y[u] * rs * bf2f(normw[pe + u]);
    }
  }
  const bool first = e0 < HD / 2;
  const int fi = first ? e0 : e0 - HD / 2;
  const float* cs = A.rope + ((size_t)p * (HD / 2) + fi) * 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float cv = cs[2 * u], sv = cs[2 * u + 1];
    out[u] = first ? x[u] * cv - y[u] * sv : x[u] * cv + y[u] * sv;
  }
}

template <int HD, int GM>
__device__ bool attn_task(const DevArgs& A, const Task& t, char* ring, float* red, Ctrl* c, CState& s, int cu, int w, int lane) {
  constexpr int LPR = HD / 8, RP = 64 / LPR, RPC = 4096 / HD;
  constexpr float kLog2e = 1.4426950408889634f;
  const int l = t.layer, G = A.G, e0 = (lane % LPR) * 8, gi = lane / LPR;
  const float qscale = kLog2e / sqrtf((float)HD);
  const long long W = attn_total(c, A.b, A.nkv);
  long long pos = cu_lo(cu, W, A.ncu), hi = cu_lo(cu + 1, W, A.ncu);
  Piece P;
  int qc = s.q, pidx = 0;
  const LayerW& lw = A.layers[l];
  const int stride_st = kComputeWaves * GM * (HD + 4);
  while (next_piece(c, A.b, A.nkv, RPC, pos, hi, P)) {
    const int p = c->slen[P.i] - 1;
    const float* qrow = A.qkv + ((size_t)l * A.bcap + P.i) * A.nqkv;
    float q[GM][8], o[GM][8];
    SoftState st[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      st[h].m = -INFINITY;
      st[h].l = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) o[h][u] = 0.f;
      if (h < G) {
        rope_head<HD>(A, qrow + (size_t)(P.g * G + h) * HD, A.qk_norm ? lw.q_norm : nullptr, p, e0, q[h]);
#pragma unroll
        for (int u = 0; u < 8; ++u) q[h][u] *= qscale;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) q[h][u] = 0.f;
      }
    }
    // cached rows, streamed by the loader
    for (int ch = 0; ch < P.nch; ++ch) {
      const int gq = qc + ch;
      if ((gq & (kComputeWaves - 1)) != w) continue;
      if (!wait_chunk(A, c, gq)) return false;
      const char* slot = ring + (size_t)(gq % A.nslot) * kChunkBytes;
      const int rows = min(RPC, P.ncached - ch * RPC);
#pragma unroll 2
      for (int pass = 0; pass < RPC / RP; ++pass) {
        const int row = pass * RP + gi;
        u32x4 kv = lds_ld16(slot + row * HD * 2 + e0 * 2);
        u32x4 vv = lds_ld16(slot + 8192 + row * HD * 2 + e0 * 2);
        float kf[8], vf[8];
        unpack8(kv, kf);
        unpack8(vv, vf);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h >= G) continue;
          float sc = 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u) sc += q[h][u] * kf[u];
#pragma unroll
          for (int m = 1; m < LPR; m <<= 1) sc += __shfl_xor(sc, m);
          if (row < rows) {
            const float mn = fmaxf(st[h].m, sc);
            const float fa = exp2f(st[h].m - mn), pw = exp2f(sc - mn);
            st[h].l = st[h].l * fa + pw;
#pragma unroll
            for (int u = 0; u < 8; ++u) o[h][u] = o[h][u] * fa + pw * vf[u];
            st[h].m = mn;
          }
        }
      }
      free_chunk(A, c, gq, lane);
    }
    // the new row: K after QK-norm + RoPE, V raw, both rounded to bf16,
    // written to the cache and absorbed by lane group 0 of wave 0
    if (w == 0 && P.has_new) {
      float kn[8], vn[8];
      const float* krow = qrow + A.qdim + (size_t)P.g * HD;
      const float* vrow = qrow + A.qdim + A.kvdim + (size_t)P.g * HD;
      rope_head<HD>(A, krow, A.qk_norm ? lw.k_norm : nullptr, p, e0, kn);
      u32x4 v0 = co_load16(vrow, (uint32_t)(e0 * 4)), v1 = co_load16(vrow, (uint32_t)((e0 + 4) * 4));
      float vr[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z), __uint_as_float(v0.w),
                     __uint_as_float(v1.x), __uint_as_float(v1.y), __uint_as_float(v1.z), __uint_as_float(v1.w)};
      u32x4 kb = {pack_bf2(kn[0], kn[1]), pack_bf2(kn[2], kn[3]), pack_bf2(kn[4], kn[5]), pack_bf2(kn[6], kn[7])};
      u32x4 vb = {pack_bf2(vr[0], vr[1]), pack_bf2(vr[2], vr[3]), pack_bf2(vr[4], vr[5]), pack_bf2(vr[6], vr[7])};
      unpack8(kb, kn);
      unpack8(vb, vn);
      if (gi == 0) {
        const size_t slot_row = ((((size_t)l * A.kv_bcap + P.i) * A.nkv + P.g) * A.kv_scap + p) * HD + e0;
        *(u32x4*)(A.kc + slot_row) = kb;
        *(u32x4*)(A.vc + slot_row) = vb;
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) continue;
        float sc = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) sc += q[h][u] * kn[u];
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) sc += __shfl_xor(sc, m);
        if (gi == 0) {
          const float mn = fmaxf(st[h].m, sc);
          const float fa = exp2f(st[h].m - mn), pw = exp2f(sc - mn);
          st[h].l = st[h].l * fa + pw;
#pragma unroll
          for (int u = 0; u < 8; ++u) o[h][u] = o[h][u] * fa + pw * vn[u];
          st[h].m = mn;
        }
      }
    }
    // merge the lane groups of this wave
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) continue;
        const float m2 = __shfl_xor(st[h].m, msk), l2 = __shfl_xor(st[h].l, msk);
        const float mn = fmaxf(st[h].m, m2);
        const float fa = mn == -INFINITY ? 0.f : exp2f(st[h].m - mn);
        const float fb = mn == -INFINITY ? 0.f : exp2f(m2 - mn);
#pragma unroll
        for (int u = 0; u < 8; ++u) o[h][u] = o[h][u] * fa + __shfl_xor(o[h][u], msk) * fb;
        st[h].l = st[h].l * fa + l2 * fb;
        st[h].m = mn;
      }
    }
    // wave states -> LDS (double-buffered by piece parity)
    float* sb = red + (pidx & 1) * stride_st + w * GM * (HD + 4);
    if (gi == 0) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) continue;
        *(f32x4*)(sb + h * (HD + 4) + e0) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
        *(f32x4*)(sb + h * (HD + 4) + e0 + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
        if (lane == 0) {
          sb[h * (HD + 4) + HD] = st[h].m;
          sb[h * (HD + 4) + HD + 1] = st[h].l;
        }
      }
    }
    if (!cbar(A, c, s.gen, lane)) return false;
    if (w == 0) {
      // merge the 4 wave states (lane group 0 holds 8 elements per lane)
      const float* s0 = red + (pidx & 1) * stride_st;
      float M[GM], Lsum[GM], O[GM][8];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        M[h] = -INFINITY;
        Lsum[h] = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) O[h][u] = 0.f;
        if (h >= G) continue;
        for (int ww = 0; ww < kComputeWaves; ++ww) {
          const float* e = s0 + ww * GM * (HD + 4) + h * (HD + 4);
          const float m2 = e[HD], l2 = e[HD + 1];
          const float mn = fmaxf(M[h], m2);
          const float fa = mn == -INFINITY ? 0.f : exp2f(M[h] - mn);
          const float fb = mn == -INFINITY ? 0.f : exp2f(m2 - mn);
#pragma unroll
          for (int u = 0; u < 8; ++u) O[h][u] = O[h][u] * fa + e[e0 + u] * fb;
          Lsum[h] = Lsum[h] * fa + l2 * fb;
          M[h] = mn;
        }
      }
      const int s_i = c->slen[P.i];
      const int c_first = cu_of(P.seg_start, W, A.ncu), c_last = cu_of(P.seg_start + s_i - 1, W, A.ncu);
      // CUs whose range is empty (fewer rows than CUs) hold no piece
      const int npieces = W >= A.ncu ? c_last - c_first + 1
                                     : (int)(cu_lo(c_last + 1, W, A.ncu) - cu_lo(c_first, W, A.ncu));
      bool finisher = npieces == 1;
      const int pstride = GM * (HD + 4);
      if (!finisher) {
        float* dst = A.apart + (size_t)(cu + P.sid) * pstride;
        if (gi == 0) {
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            if (h >= G) continue;
            co_store16(dst, (uint32_t)((h * (HD + 4) + e0) * 4),
                       u32x4{__float_as_uint(O[h][0]), __float_as_uint(O[h][1]), __float_as_uint(O[h][2]), __float_as_uint(O[h][3])});
            co_store16(dst, (uint32_t)((h * (HD + 4) + e0 + 4) * 4),
                       u32x4{__float_as_uint(O[h][4]), __float_as_uint(O[h][5]), __float_as_uint(O[h][6]), __float_as_uint(O[h][7])});
            if (lane == 0) co_store8(dst, (uint32_t)((h * (HD + 4) + HD) * 4), u32x2{__float_as_uint(M[h]), __float_as_uint(Lsum[h])});
          }
        }
        wait_mem();
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(A.seg_ctr + P.sid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        finisher = (int)old == npieces - 1;
        if (finisher) {
          if (lane == 0) __hip_atomic_store(A.seg_ctr + P.sid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            M[h] = -INFINITY;
            Lsum[h] = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) O[h][u] = 0.f;
            if (h >= G) continue;
            for (int cc = c_first; cc <= c_last; ++cc) {
              if (W < A.ncu && cu_lo(cc + 1, W, A.ncu) == cu_lo(cc, W, A.ncu)) continue;
              const float* src = A.apart + (size_t)(cc + P.sid) * pstride + h * (HD + 4);
              u32x4 a0 = co_load16(src, (uint32_t)(e0 * 4)), a1 = co_load16(src, (uint32_t)((e0 + 4) * 4));
              const float m2 = co_loadf(src, HD * 4), l2 = co_loadf(src, (HD + 1) * 4);
              const float mn = fmaxf(M[h], m2);
              const float fa = mn == -INFINITY ? 0.f : exp2f(M[h] - mn);
              const float fb = mn == -INFINITY ? 0.f : exp2f(m2 - mn);
              float ov[8] = {__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z), __uint_as_float(a0.w),
                             __uint_as_float(a1.x), __uint_as_float(a1.y), __uint_as_float(a1.z), __uint_as_float(a1.w)};
#pragma unroll
              for (int u = 0; u < 8; ++u) O[h][u] = O[h][u] * fa + ov[u] * fb;
              Lsum[h] = Lsum[h] * fa + l2 * fb;
              M[h] = mn;
            }
          }
        }
      }
      if (finisher && gi == 0) {
        uint16_t* ob = A.attn_out + ((size_t)l * A.bcap + P.i) * A.qdim;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h >= G) continue;
          const float inv = 1.0f / Lsum[h];
          co_store16(ob, (uint32_t)((((size_t)(P.g * G + h)) * HD + e0) * 2),
                     u32x4{pack_bf2(O[h][0] * inv, O[h][1] * inv), pack_bf2(O[h][2] * inv, O[h][3] * inv),
                           pack_bf2(O[h][4] * inv, O[h][5] * inv), pack_bf2(O[h][6] * inv, O[h][7] * inv)});
        }
      }
    }
    qc += P.nch;
    ++pidx;
  }
  wait_mem();
  if (!cbar(A, c, s.gen, lane)) return false;
  if (w == 0 && lane == 0) signal_counter(A, t.signal_ctr, cu);
  return true;
}

template <int HD>
__device__ __forceinline__ bool attn_dispatch(const DevArgs& A, const Task& t, char* ring, float* red, Ctrl* c, CState& s, int cu, int w, int lane) {
  if (A.G <= 1) return attn_task<HD, 1>(A, t, ring, red, c, s, cu, w, lane);
  if (A.G <= 2) return attn_task<HD, 2>(A, t, ring, red, c, s, cu, w, lane);
  if (A.G <= 4) return attn_task<HD, 4>(A, t, ring, red, c, s, cu, w, lane);
  return attn_task<HD, 8>(A, t, ring, red, c, s, cu, w, lane);
}

__device__ bool gemv_dispatch(const DevArgs& A, const Task& t, char* ring, char* xb, float* red, Ctrl* c, CState& s, int cu, int w, int lane) {
  if (A.mfma) {
    if (t.nsub == 4) return gemv_task<1, 4>(A, t, ring, xb, red, c, s, cu, w, lane);
    if (t.nsub == 2) return gemv_task<1, 2>(A, t, ring, xb, red, c, s, cu, w, lane);
    return gemv_task<1, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
  }
  switch (A.b) {
    case 1: return gemv_task<1, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    case 2: return gemv_task<2, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    case 3: return gemv_task<3, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    case 4: return gemv_task<4, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    case 5: return gemv_task<5, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    case 6: return gemv_task<6, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
    default: return gemv_task<7, 1>(A, t, ring, xb, red, c, s, cu, w, lane);
  }
}

__device__ void compute_main(const DevArgs& A, char* ring, char* xb, float* red, Ctrl* c, int cu, int w, int lane) {
  const Task* T = A.tasks + A.task_off[cu];
  const int nt = A.task_off[cu + 1] - A.task_off[cu];
  CState s{0, 0, -1, -1, -1, -1, -1};
  const int rpc = 4096 / A.hd;
  bool had_lm = false;
  for (int ti = 0; ti < nt; ++ti) {
    const Task t = T[ti];
    if (t.wait_ctr >= 0 && t.wait_ctr != s.last_dep) {
      if (w == 0) {
        if (!wait_counter(A, c, t.wait_ctr, lane)) return;
        if (lane == 0) lds_st_rel(&c->dep, ti + 1);
      } else {
        Spin sp = spin_start();
        while (lds_ld_acq(&c->dep) < ti + 1)
          if (!spin_ok(A, c, sp)) return;
      }
      s.last_dep = t.wait_ctr;
    }
    bool ok;
    int nch = 0;
    if (t.type == TT_GEMV) {
      ok = gemv_dispatch(A, t, ring, xb, red, c, s, cu, w, lane);
      nch = t.nchunks;
      had_lm = had_lm || t.stage == ST_LM;
    } else if (t.type == TT_ATTN) {
      ok = A.hd == 128 ? attn_dispatch<128>(A, t, ring, red, c, s, cu, w, lane)
                       : attn_dispatch<64>(A, t, ring, red, c, s, cu, w, lane);
      nch = attn_task_chunks(A, c, cu, rpc);
    } else {
      ok = embed_task(A, t, c, s, cu, w, lane);
    }
    if (!ok) return;
    s.q += nch;
  }
  // Greedy tokens: once every LM task has signalled, the argmax keys are
  // final.  Every CU that ran LM tasks checks once; the CU whose signal was
  // the last one is guaranteed to see completion (duplicates write the same
  // values).
  if (w == 0 && had_lm && A.next_tokens) {
    wait_mem();
    const int ctr = ctr_lm(A.L);
    const uint32_t* p = bank_ptr(A, A.bank) + lane * A.ctr_stride + ctr;
    int v = (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(v >= A.expect[ctr * kShards + lane]) && lane < A.b) {
      unsigned long long key = __hip_atomic_load(keys_ptr(A) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      A.next_tokens[lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void mk_step_kernel(DevArgs A) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* ring = lds;
  char* xb = lds + (size_t)A.nslot * kChunkBytes;
  float* red = (float*)(xb + A.xb_bytes);
  Ctrl* c = (Ctrl*)((char*)red + kRedBytes);
  const int cu = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  // zero this CU's slice of the bank the next step will use
  {
    uint32_t* nb = bank_ptr(A, A.bank ^ 1);
    const int per = (A.bank_words + A.ncu - 1) / A.ncu;
    const int lo = cu * per, hi = min(A.bank_words, lo + per);
    for (int i = lo + tid; i < hi; i += kThreads) nb[i] = 0u;
  }
  if (tid < kMaxSlots) {
    c->ready[tid] = 0;
    c->freed[tid] = 0;
  }
  if (tid == 0) {
    c->dep = 0;
    c->bar = 0;
    c->fin = 0;
    c->abort = 0;
  }
  // per-sequence inputs, validated and clamped identically on every CU
  if (tid < A.b) {
    uint32_t st = 0;
    int tok = A.tokens[tid];
    if (tok < 0 || tok >= A.V) {
      st |= 1u;
      tok = tok < 0 ? 0 : A.V - 1;
    }
    int p = A.positions[tid];
    const int cap = min(A.max_seq, A.kv_scap);
    if (p < 0 || p >= cap) {
      st |= 2u;
      p = p < 0 ? 0 : cap - 1;
    }
    if (A.seq_lens[tid] != A.positions[tid] + 1) st |= 4u;
    c->tok[tid] = tok;
    c->pos[tid] = p;
    c->slen[tid] = p + 1;
    if (st && cu == 0) atomicOr(A.status, st);
  }
  __syncthreads();
  if (w < kComputeWaves) compute_main(A, ring, xb, red, c, cu, w, lane);
  else loader_main(A, ring, c, cu, w - kComputeWaves, lane);
}

size_t lds_bytes(int nslot, int xb_bytes) {
  return (size_t)nslot * kChunkBytes + xb_bytes + kRedBytes + sizeof(Ctrl);
}

hipError_t launch_step(const DevArgs& A, hipStream_t stream) {
  const size_t lds = lds_bytes(A.nslot, A.xb_bytes);
  hipError_t e = hipFuncSetAttribute((const void*)mk_step_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mk_step_kernel, dim3(A.ncu), dim3(kThreads), lds, stream, A);
  return hipGetLastError();
}

}  // namespace mk
