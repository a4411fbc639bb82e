"""Host-side checks of the C-ABI library: it loads without a GPU, exports
every entry point include/mk.h declares, rejects bad arguments before touching
the device, and its schedule builder validates every workload."""
import ctypes
import os
import re

import pytest

from decode_megakernel_amd import binding
from mkinputs import WORKLOADS, TINY_LLAMA, TINY_QWEN, SMALL_LLAMA_H64, SMALL_QWEN_H128, SMALL_MHA_H128

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mk_\w+)\s*\(", src, re.M)))


def test_header_declares_expected_entry_points():
    assert declared_entry_points() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    for name in declared_entry_points():
        assert hasattr(lib, name), name


def test_error_strings():
    lib = binding.lib()
    assert lib.mk_error_string(0) == b"ok"
    assert lib.mk_error_string(-2) == b"unsupported model shape"


def _cfg(shape, **kw):
    c = binding.model_cfg(shape, 4, 256)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_create_rejects_bad_arguments_before_the_device():
    lib = binding.lib()
    h = ctypes.c_void_p()
    wp = binding.WeightPtrs()
    assert lib.mk_create(None, ctypes.byref(wp), ctypes.byref(h)) == -1
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA)), None, ctypes.byref(h)) == -1
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA)), ctypes.byref(wp), ctypes.byref(h)) == -1  # NULL weights
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA, head_dim=32)), ctypes.byref(wp), ctypes.byref(h)) == -2
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA, hidden=200)), ctypes.byref(wp), ctypes.byref(h)) == -2
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA, max_batch=17)), ctypes.byref(wp), ctypes.byref(h)) == -1
    assert lib.mk_create(ctypes.byref(_cfg(TINY_LLAMA, n_q_heads=5)), ctypes.byref(wp), ctypes.byref(h)) == -1
    assert not h.value


def test_step_rejects_null_handle_and_bad_batch():
    lib = binding.lib()
    assert lib.mk_decode_step(None, 1, None, None, None, None, None, None, None) == -1
    assert lib.mk_get_status(None, None, None) == -1
    assert lib.mk_destroy(None) == -1


SHAPES = [TINY_LLAMA, TINY_QWEN, SMALL_LLAMA_H64, SMALL_QWEN_H128, SMALL_MHA_H128]


@pytest.mark.parametrize("key", sorted(WORKLOADS))
def test_plan_validates_workloads(key):
    w = WORKLOADS[key]
    for b in sorted({p.batch for p in w.phases} | {1, 16}):
        st = binding.plan(w.shape, b, 256, max_batch=16)
        assert st["mfma"] == (1 if b >= 8 else 0)
        # every weight byte of every layer and the LM head is streamed exactly once
        sh = w.shape
        per_layer = 2 * sh.hidden * (sh.q_dim + 2 * sh.kv_dim) + 2 * sh.q_dim * sh.hidden + 6 * sh.hidden * sh.intermediate
        assert st["weight_bytes"] == sh.n_layers * per_layer + 2 * sh.vocab * sh.hidden


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_plan_small_shapes_all_batches(shape):
    for b in range(1, 17):
        for ncu in (1, 7, 256):
            st = binding.plan(shape, b, ncu, max_batch=16)
            assert st["n_tasks"] > 0


def test_plan_rejects_batch_over_capacity():
    with pytest.raises(binding.MKError):
        binding.plan(TINY_LLAMA, 5, 256, max_batch=4)


@pytest.mark.parametrize("permute", [True, False])
def test_paged_pools_hold_the_contiguous_rows(permute):
    """The benchmark's paged pools: block table entry j of row i names the
    pool block that holds positions j*block .. of sequence i, bit for bit the
    rows of the contiguous cache; the block ids are a permutation."""
    import torch
    from mkinputs import make_kv_cache, make_paged_kv
    from mkinputs.configs import SMALL_MHA_H64 as sh
    ctx, B, S, bs = [100, 300, 5], 3, 512, 128
    K, V = make_kv_cache(sh, 7, ctx, B, S)
    Kp, Vp, bt = make_paged_kv(sh, 7, ctx, B, S, bs, permute=permute)
    assert sorted(bt.flatten().tolist()) == list(range(B * S // bs))
    if not permute:
        assert bt.flatten().tolist() == list(range(B * S // bs))
    for l in range(sh.n_layers):
        for i in range(B):
            for j in range(S // bs):
                blk = int(bt[i, j])
                assert torch.equal(Kp[l, blk].view(torch.int16), K[l, i, :, j * bs:(j + 1) * bs].view(torch.int16))
                assert torch.equal(Vp[l, blk].view(torch.int16), V[l, i, :, j * bs:(j + 1) * bs].view(torch.int16))
