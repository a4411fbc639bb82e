"""ctypes binding of the C ABI in include/mk.h.

Argument marshalling only: every step of the decode runs in the HIP kernel of
libmk.so.  If the library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
STATUS_BAD_TOKEN = 1
STATUS_BAD_POSITION = 2
STATUS_BAD_SEQLEN = 4
STATUS_TIMEOUT = 8
STATUS_BAD_BLOCK = 16
ERRORS = {-1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_UNSUPPORTED", -3: "MK_ERR_OOM", -4: "MK_ERR_HIP",
          -5: "MK_ERR_PLAN", -6: "MK_ERR_TOO_LARGE"}


class MKError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERRORS.get(code, code)}")
        self.code = code


class ModelCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float), ("max_batch", ctypes.c_int32),
                ("max_seq", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class WeightPtrs(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("q_proj", _PP), ("k_proj", _PP), ("v_proj", _PP), ("o_proj", _PP),
                ("q_norm", _PP), ("k_norm", _PP), ("mlp_norm", _PP), ("gate_proj", _PP), ("up_proj", _PP),
                ("down_proj", _PP)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("batch_cap", ctypes.c_int32),
                ("seq_cap", ctypes.c_int32)]


class PagedKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("n_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


class TaskInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("type", "stage", "layer", "row0", "nsub", "k0", "k1", "ks", "nks",
                                              "group", "part_slot", "nchunks", "flags")]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int32), ("max_tasks_per_cu", ctypes.c_int32),
                ("n_counters", ctypes.c_int32), ("mfma", ctypes.c_int32), ("weight_bytes", ctypes.c_int64),
                ("max_cu_weight_bytes", ctypes.c_int64), ("stage_balance_min", ctypes.c_double),
                ("stage_tasks", ctypes.c_int32 * 6), ("stage_ksplit", ctypes.c_int32 * 6),
                ("stage_rows_per_task", ctypes.c_int32 * 6), ("stage_cus", ctypes.c_int32 * 6),
                ("stage_shared_prev", ctypes.c_int32 * 6), ("attn_slot_cap", ctypes.c_int32),
                ("attn_slots_valid", ctypes.c_int32), ("stage_kpieces", ctypes.c_int32 * 6)]


EXPORTS = ["mk_create", "mk_decode_step", "mk_decode_step_paged", "mk_decode_step_static", "mk_copy_hidden", "mk_copy_state", "mk_copy_trace", "mk_get_status",
           "mk_reset", "mk_set_context_bound", "mk_set_midstate_dump", "mk_destroy", "mk_error_string", "mk_plan", "mk_plan_streams"]
STATE_HIDDEN, STATE_HMID, STATE_QKV, STATE_ATTN, STATE_ACT = 0, 1, 2, 3, 4
STAT_WORDS = 80  # per-CU trace totals, see mk_copy_trace

_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m decode_megakernel_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.mk_create.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(WeightPtrs), ctypes.POINTER(vp)]
    L.mk_decode_step.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp]
    L.mk_decode_step_static.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp]
    L.mk_decode_step_paged.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(PagedKV), vp, vp, vp]
    L.mk_copy_hidden.argtypes = [vp, i32, vp, vp]
    L.mk_copy_state.argtypes = [vp, i32, i32, vp, vp]
    L.mk_copy_trace.argtypes = [vp, vp, ctypes.c_int64, ctypes.POINTER(i32), ctypes.POINTER(i32), vp]
    L.mk_get_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    L.mk_reset.argtypes = [vp, vp]
    L.mk_set_midstate_dump.argtypes = [vp, vp]
    L.mk_set_context_bound.argtypes = [vp, i32]
    L.mk_destroy.argtypes = [vp]
    L.mk_error_string.argtypes = [ctypes.c_int]
    L.mk_error_string.restype = ctypes.c_char_p
    L.mk_plan.argtypes = [ctypes.POINTER(ModelCfg), i32, i32, ctypes.POINTER(PlanStats)]
    L.mk_plan_streams.argtypes = [ctypes.POINTER(ModelCfg), i32, i32, ctypes.POINTER(TaskInfo), i32,
                                  ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    for name in EXPORTS:
        if name != "mk_error_string":
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != MK_OK:
        raise MKError(rc, what)


def model_cfg(shape, max_batch: int, max_seq: int) -> ModelCfg:
    return ModelCfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                    shape.intermediate, shape.vocab, int(shape.tied_embeddings), int(shape.qk_norm),
                    float(shape.rope_theta), float(shape.rms_eps), int(max_batch), int(max_seq))


def plan(shape, batch: int, n_cu: int = 256, max_batch: int = 16, max_seq: int = 8192) -> dict:
    """Build and validate the per-CU schedule on the host (no GPU)."""
    st = PlanStats()
    cfg = model_cfg(shape, max_batch, max_seq)
    _check(lib().mk_plan(ctypes.byref(cfg), int(batch), int(n_cu), ctypes.byref(st)), "mk_plan")
    out = {k: getattr(st, k) for k, _ in PlanStats._fields_}
    for k in ("stage_tasks", "stage_ksplit", "stage_rows_per_task", "stage_cus", "stage_shared_prev",
              "stage_kpieces"):
        out[k] = list(out[k])
    return out


def torch_float32():
    import torch
    return torch.float32


def plan_streams(shape, batch: int, n_cu: int, max_batch: int = 16, max_seq: int = 8192):
    """The per-CU instruction streams (host only): (list of per-CU lists of task
    dicts, attention slot map [n_layers][n_cu + 1])."""
    cfg = model_cfg(shape, max_batch, max_seq)
    n = ctypes.c_int32()
    offs = (ctypes.c_int32 * (n_cu + 1))()
    rc = lib().mk_plan_streams(ctypes.byref(cfg), int(batch), int(n_cu), None, 0, offs, None, ctypes.byref(n))
    if rc != MK_OK and n.value <= 0:
        _check(rc, "mk_plan_streams")
    tasks = (TaskInfo * n.value)()
    amap = (ctypes.c_int32 * (shape.n_layers * (n_cu + 1)))()
    _check(lib().mk_plan_streams(ctypes.byref(cfg), int(batch), int(n_cu), tasks, n.value, offs, amap,
                                 ctypes.byref(n)), "mk_plan_streams")
    names = [f for f, _ in TaskInfo._fields_]
    streams = [[{k: getattr(tasks[i], k) for k in names} for i in range(offs[c], offs[c + 1])] for c in range(n_cu)]
    L = shape.n_layers
    return streams, [list(amap[l * (n_cu + 1):(l + 1) * (n_cu + 1)]) for l in range(L)]


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class DecodeEngine:
    """Owns one mk_handle; the caller owns weights, KV cache and step buffers.

    `weights` maps Hugging Face names to contiguous bf16 CUDA tensors.
    """

    def __init__(self, shape, weights: dict, max_batch: int, max_seq: int):
        self.shape = shape
        self._keep = []   # ctypes arrays that the C side reads during mk_create
        L = shape.n_layers

        def ptr(name):
            t = weights[name]
            assert t.is_cuda and t.is_contiguous(), name
            return t.data_ptr()

        def arr(suffix, optional=False):
            if optional and not shape.qk_norm:
                return ctypes.cast(None, _PP)
            a = (ctypes.c_void_p * L)(*[ptr(f"model.layers.{l}.{suffix}") for l in range(L)])
            self._keep.append(a)
            return ctypes.cast(a, _PP)

        wp = WeightPtrs(
            ptr("model.embed_tokens.weight"),
            None if shape.tied_embeddings else ptr("lm_head.weight"),
            ptr("model.norm.weight"),
            arr("input_layernorm.weight"), arr("self_attn.q_proj.weight"), arr("self_attn.k_proj.weight"),
            arr("self_attn.v_proj.weight"), arr("self_attn.o_proj.weight"),
            arr("self_attn.q_norm.weight", True), arr("self_attn.k_norm.weight", True),
            arr("post_attention_layernorm.weight"), arr("mlp.gate_proj.weight"), arr("mlp.up_proj.weight"),
            arr("mlp.down_proj.weight"))
        self.cfg = model_cfg(shape, max_batch, max_seq)
        h = ctypes.c_void_p()
        _check(lib().mk_create(ctypes.byref(self.cfg), ctypes.byref(wp), ctypes.byref(h)), "mk_create")
        self.handle = h
        self.max_batch = max_batch

    def step(self, tokens, positions, seq_lens, k_cache, v_cache, logits, next_tokens=None, stream=None,
             batch=None, static=False):
        """Enqueue one decode step; all tensors are CUDA tensors the caller owns.

        k_cache, v_cache: bf16 [L][batch_cap][n_kv][seq_cap][hd]; tokens, positions,
        seq_lens: int32 [>= batch]; logits: float32 [>= batch, vocab].  static=True
        calls the allocation-free entry point (scratch in the library's static array)."""
        b = int(tokens.numel()) if batch is None else int(batch)
        kv = KVCache(k_cache.data_ptr(), v_cache.data_ptr(), int(k_cache.shape[1]), int(k_cache.shape[3]))
        fn = lib().mk_decode_step_static if static else lib().mk_decode_step
        rc = fn(self.handle, b, tokens.data_ptr(), positions.data_ptr(), seq_lens.data_ptr(),
                ctypes.byref(kv), logits.data_ptr(), None if next_tokens is None else next_tokens.data_ptr(),
                _stream_handle(stream))
        _check(rc, "mk_decode_step_static" if static else "mk_decode_step")

    def step_paged(self, tokens, positions, seq_lens, k_pool, v_pool, block_table, logits, next_tokens=None,
                   stream=None, batch=None):
        """Enqueue one decode step over a paged KV cache: k_pool, v_pool bf16
        [L][n_blocks][n_kv][block_size][hd]; block_table int32 [>= batch, max_blocks]
        (contiguous rows)."""
        b = int(tokens.numel()) if batch is None else int(batch)
        assert block_table.is_contiguous() and block_table.dtype.itemsize == 4
        kv = PagedKV(k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(), int(k_pool.shape[1]),
                     int(k_pool.shape[3]), int(block_table.shape[1]))
        rc = lib().mk_decode_step_paged(self.handle, b, tokens.data_ptr(), positions.data_ptr(),
                                        seq_lens.data_ptr(), ctypes.byref(kv), logits.data_ptr(),
                                        None if next_tokens is None else next_tokens.data_ptr(),
                                        _stream_handle(stream))
        _check(rc, "mk_decode_step_paged")

    def copy_hidden(self, batch: int, out, stream=None):
        _check(lib().mk_copy_hidden(self.handle, int(batch), out.data_ptr(), _stream_handle(stream)),
               "mk_copy_hidden")

    def copy_state(self, which: int, batch: int, out, stream=None):
        _check(lib().mk_copy_state(self.handle, int(which), int(batch), out.data_ptr(), _stream_handle(stream)),
               "mk_copy_state")

    def state(self, which: int, batch: int):
        """Mid-state buffer of the last step as a new CUDA tensor [layers, batch, width]."""
        import torch
        sh = self.shape
        L = sh.n_layers
        spec = {STATE_HIDDEN: (L + 1, sh.hidden, torch.float32), STATE_HMID: (L, sh.hidden, torch.float32),
                STATE_QKV: (L, sh.q_dim + 2 * sh.kv_dim, torch.float32),
                STATE_ATTN: (L, sh.q_dim, torch.float32), STATE_ACT: (L, sh.intermediate, torch.float32)}
        nl, width, dt = spec[which]
        out = torch.empty((nl, batch, width), dtype=dt, device="cuda")
        self.copy_state(which, batch, out)
        return out

    def trace(self):
        """(per-task records [n_cu, cap, 4] uint64, per-CU wait stats [n_cu, 32] uint64) of
        the last step, or None when the handle was created without MK_TRACE."""
        import torch
        n_cu, cap = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().mk_copy_trace(self.handle, None, 0, ctypes.byref(n_cu), ctypes.byref(cap), None),
               "mk_copy_trace")
        if cap.value <= 0:
            return None
        n, c = n_cu.value, cap.value
        buf = torch.empty(n * c * 4 + n * STAT_WORDS, dtype=torch.int64, device="cuda")
        _check(lib().mk_copy_trace(self.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel() * 8,
                                   ctypes.byref(n_cu), ctypes.byref(cap), _stream_handle(None)), "mk_copy_trace")
        arr = buf.cpu().numpy().view("uint64")
        return arr[: n * c * 4].reshape(n, c, 4), arr[n * c * 4:].reshape(n, STAT_WORDS)

    def status(self, stream=None) -> int:
        s = ctypes.c_uint32()
        _check(lib().mk_get_status(self.handle, _stream_handle(stream), ctypes.byref(s)), "mk_get_status")
        return int(s.value)

    def set_context_bound(self, max_seq_len: int):
        """Route later steps to the attention partition of their context bucket
        (0: no bound)."""
        _check(lib().mk_set_context_bound(self.handle, int(max_seq_len)), "mk_set_context_bound")

    def set_midstate_dump(self, out):
        """Every later step also writes its residual stream into `out` (a CUDA
        float32 tensor [n_layers+1, max_batch, hidden] the caller keeps alive);
        None switches it off."""
        if out is not None:
            assert out.is_cuda and out.dtype == torch_float32() and out.is_contiguous()
            assert tuple(out.shape) == (self.shape.n_layers + 1, self.max_batch, self.shape.hidden)
        _check(lib().mk_set_midstate_dump(self.handle, None if out is None else out.data_ptr()),
               "mk_set_midstate_dump")
        self._dump = out

    def reset(self, stream=None):
        _check(lib().mk_reset(self.handle, _stream_handle(stream)), "mk_reset")

    def close(self):
        if getattr(self, "handle", None):
            lib().mk_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
