"""The C ABI on the host: the library loads, exports every symbol the header
declares, and its validation returns the documented codes (no GPU needed:
nothing here reaches a HIP call)."""
import ctypes as C

import pytest

import synth
from speculative_decoding_rvq_amd import binding


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_every_header_symbol_is_exported(L):
    syms = binding.header_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(binding._SIGS)


def test_workspace_sizes():
    for cid in synth.WORKLOADS:
        n = binding.workspace_bytes(binding.make_cfg(synth.config(cid)))
        assert n > 0 and n % 256 == 0, cid
    n1 = binding.workspace_bytes(binding.make_cfg(synth.config("tiny-64"),
                                                  max_streams=1))
    n64 = binding.workspace_bytes(binding.make_cfg(synth.config("tiny-64")))
    assert n64 > n1


def _create(cfg):
    h = C.c_void_p()
    w = binding.Weights(1, 1, 1, C.cast((C.c_void_p * 18)(*([1] * 18)),
                                        C.POINTER(C.c_void_p)))
    rc = binding.lib().cp_spec_create(C.byref(w), C.byref(cfg), None, 0,
                                      C.byref(h))
    return rc, binding.last_error()


@pytest.mark.parametrize("field,value,code,msg", [
    ("verify_size", 1, binding.EINVAL, "no draft slot"),
    ("verify_size", 9, binding.EINVAL, "0 (off) or 2..8"),
    ("verify_size", -1, binding.EINVAL, "0 (off) or 2..8"),
    ("vocab", 8192, binding.EUNSUPPORTED, "small-vocabulary"),
    ("vocab", 300, binding.EUNSUPPORTED, "256 * 2^i"),
    ("top_k", 0, binding.EINVAL, "top_k"),
    ("top_k", 257, binding.EINVAL, "top_k"),
    ("temperature", 0.0, binding.EINVAL, "temperature"),
    ("q_heads", 3, binding.EINVAL, "multiple of kv_heads"),
    ("code_groups", 1, binding.EINVAL, "code_groups"),
    ("code_groups", 33, binding.EUNSUPPORTED, "code_groups"),
    ("hidden", 100, binding.EUNSUPPORTED, "not tileable"),
    ("max_streams", 0, binding.EINVAL, "non-positive"),
    ("head_dim", 256, binding.EUNSUPPORTED, "head_dim"),
    ("head_dim", 48, binding.EUNSUPPORTED, "head_dim"),
    ("draft_offsets", 9, binding.EINVAL, "draft_offsets"),
    ("draft_offsets", -1, binding.EINVAL, "draft_offsets"),
])
def test_create_validation(field, value, code, msg):
    cfg = binding.make_cfg(synth.config("tiny"))
    setattr(cfg, field, value)
    rc, err = _create(cfg)
    assert rc == code and msg in err, (rc, err)
    assert binding.lib().cp_spec_workspace_bytes(C.byref(cfg)) == 0


def test_greedy_ignores_sampling_fields():
    cfg = binding.make_cfg(synth.config("tiny-greedy"))
    cfg.top_k = 0
    cfg.temperature = 0.0
    assert binding.workspace_bytes(cfg) > 0


def test_workspace_checks_before_any_device_work():
    cfg = binding.make_cfg(synth.config("tiny"))
    rc, err = _create(cfg)                     # null workspace
    assert rc == binding.EWORKSPACE and "workspace" in err
    h = C.c_void_p()
    w = binding.Weights(1, 1, 1, C.cast((C.c_void_p * 18)(*([1] * 18)),
                                        C.POINTER(C.c_void_p)))
    n = binding.workspace_bytes(cfg)
    rc = binding.lib().cp_spec_create(C.byref(w), C.byref(cfg),
                                      C.c_void_p(0x1000 + 3), n, C.byref(h))
    assert rc == binding.EWORKSPACE and "aligned" in binding.last_error()
    rc = binding.lib().cp_spec_create(C.byref(w), C.byref(cfg),
                                      C.c_void_p(0x1000), n - 1, C.byref(h))
    assert rc == binding.EWORKSPACE


def test_null_handle_calls_are_rejected():
    Lb = binding.lib()
    assert Lb.cp_spec_decode_frames(None, None, 1, 1, None, None, None, None,
                                    None, None) == binding.EINVAL
    assert Lb.cp_spec_topk_sample(None, None, 1, None, None, None, None,
                                  None) == binding.EINVAL
    Lb.cp_spec_destroy(None)


def test_draft_offsets_workspace_and_pointer_checks():
    c = synth.config("qwen3tts")
    base = binding.workspace_bytes(binding.make_cfg(c))
    cfg = binding.make_cfg(c)
    cfg.draft_offsets = 3
    n = binding.workspace_bytes(cfg)
    # one [B][N-1][H] float32 buffer of draft input rows
    W = c["verify_size"] - 1
    assert n - base == (W * c["hidden"] * 4 + 255) // 256 * 256
    # speculation off: no drafts, no buffer
    cfg0 = binding.make_cfg(c)
    cfg0.verify_size = 0
    cfg0.draft_offsets = 3
    cfg1 = binding.make_cfg(c)
    cfg1.verify_size = 0
    assert binding.workspace_bytes(cfg0) == binding.workspace_bytes(cfg1)
    layer = C.cast((C.c_void_p * (9 * c["layers"]))(*([1] * 9 * c["layers"])),
                   C.POINTER(C.c_void_p))
    h = C.c_void_p()
    for ptr in (None, 0x1004):  # missing, misaligned
        w = binding.Weights(1, 1, 1, layer, ptr)
        rc = binding.lib().cp_spec_create(C.byref(w), C.byref(cfg),
                                          C.c_void_p(0x1000), n, C.byref(h))
        assert rc == binding.EINVAL and "draft_offsets" in binding.last_error()


def _tree_cfg(parents, **over):
    c = synth.config("tiny", **over)
    cfg = binding.make_cfg(dict(c, tree=parents))
    return cfg


@pytest.mark.parametrize("parents,over,code,msg", [
    ([0] * 64, {}, binding.EINVAL, "tree_nodes"),
    ([0, 2], {}, binding.EINVAL, "tree_parent"),
    ([1], {}, binding.EINVAL, "tree_parent"),
    (list(range(8)), {}, binding.EINVAL, "tree depth"),
    ([0, 0], {"fused_draft": 1}, binding.EUNSUPPORTED, "chain windows only"),
])
def test_tree_validation(parents, over, code, msg):
    cfg = _tree_cfg(parents, **over)
    rc, err = _create(cfg)
    assert rc == code and msg in err, (rc, err)
    assert binding.lib().cp_spec_workspace_bytes(C.byref(cfg)) == 0


@pytest.mark.parametrize("parents,over", [
    ([0] * 63, {}),                          # 63 children of the root
    (list(range(7)), {}),                    # depth 7
    ([0, 0, 1, 1], {"greedy": True}),        # greedy trees
    ([0, 0, 1, 1], {"streams": 64}),         # any stream count
])
def test_tree_shapes_accepted(parents, over):
    cfg = _tree_cfg(parents, **over)
    assert binding.lib().cp_spec_workspace_bytes(C.byref(cfg)) > 0, binding.last_error()


def test_tree_workspace_holds_node_slots():
    c = synth.config("tiny")
    n0 = binding.workspace_bytes(binding.make_cfg(c))
    n1 = binding.workspace_bytes(binding.make_cfg(dict(c, tree=[0, 0, 1, 2])))
    assert n1 > n0  # four more K/V slots per stream, five verify rows


def test_accept_noalloc_validation(L):
    """The allocation-free accept rejects bad sizes on the host, before any
    HIP call."""
    f = L.cp_spec_accept_noalloc
    one = C.c_void_p(16)
    args = [one] * 9
    assert f(None, 300, 0, 1, 3, *args) == binding.EINVAL
    assert "vocab" in binding.last_error()
    assert f(None, 256, 0, 8193, 7, *args) == binding.EINVAL
    assert "static scratch" in binding.last_error()
    assert f(None, 256, 0, 1, 8, *args) == binding.EINVAL
    assert f(None, 256, 0, 0, 3, *args) == binding.OK  # nothing to do
