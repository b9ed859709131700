"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infllmv2.h")


@pytest.fixture(scope="module")
def t():
    import trainable_block_sparse_infllm_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from trainable_block_sparse_infllm_amd import build
        build.build()
    pkg.lib()
    return pkg


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"INFLLMV2_API\s+[\w\s\*]*?\b(infllmv2_\w+)\s*\(", src)))


def test_header_declares_the_binding_exports(t):
    assert declared_functions() == sorted(t.EXPORTS)


def test_library_exports_every_declared_symbol(t):
    out = subprocess.run(["nm", "-D", "--defined-only", t.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (infllmv2_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported
    for name in declared_functions():
        assert hasattr(t.lib(), name)


def test_internal_symbols_are_hidden(t):
    out = subprocess.run(["nm", "-D", "--defined-only", t.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "launch_attn_rows" not in out and "launch_decode" not in out


def cfg_ok(t, **kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, top_k=16, dense_threshold=1024)
    base.update(kw)
    return t.make_cfg(**base)


A = 0x10000   # 16-byte aligned fake device addresses: never dereferenced on a rejected call
B = 0x20000


def call(t, name, *args):
    import ctypes
    fn = getattr(t.lib(), name)
    args = [ctypes.byref(a) if hasattr(a, "_fields_") else a for a in args]
    return fn(*args), t.infllmv2_last_error()


CASES = [
    # (entry point, cfg overrides, args after cfg, expected status, message fragment)
    ("infllmv2_pool_kernels", None, (A, 64, 64, 0, B, None), -1, "cfg is NULL"),
    ("infllmv2_pool_kernels", {}, (None, 64, 64, 0, B, None), -1, "k is NULL"),
    ("infllmv2_pool_kernels", {}, (A + 2, 64, 64, 0, B, None), -1, "aligned"),
    ("infllmv2_pool_kernels", {}, (A, 64, 65, 0, B, None), -1, "exceeds kv_cap"),
    ("infllmv2_pool_kernels", {}, (A, 128, 128, 3, B, None), -1, "first_block"),
    ("infllmv2_pool_kernels", dict(n_q_heads=30), (A, 64, 64, 0, B, None), -1, "multiple"),
    ("infllmv2_pool_kernels", dict(head_dim=96), (A, 64, 64, 0, B, None), -2, "head_dim"),
    ("infllmv2_pool_kernels", dict(block_size=128), (A, 128, 128, 0, B, None), -2, "block 64"),
    ("infllmv2_pool_kernels", dict(kernel_size=33), (A, 64, 64, 0, B, None), -1, "geometry"),
    ("infllmv2_pool_kernels", dict(n_q_heads=24, n_kv_heads=1), (A, 64, 64, 0, B, None), -2, "divide 16"),
    ("infllmv2_score_blocks", {}, (A, 0, 0, 0, B, 64, A, None), -1, "n_q"),
    ("infllmv2_score_blocks", {}, (A, 1, -1, 0, B, 64, A, None), -1, "q_pos0"),
    ("infllmv2_score_blocks", {}, (A, 1, 640, 0, B, 64, A, None), -1, "beyond kv_cap"),
    ("infllmv2_score_blocks", {}, (A, 65, 0, 1, B, 8192, A, None), -1, "64 nodes"),
    ("infllmv2_score_blocks", {}, (A, 1, 0, 0, B, 64, A + 2, None), -1, "scores"),
    ("infllmv2_topk_blocks", dict(top_k=0), (A, None, None, 1, 0, 0, 64, B, None), -1, "top_k"),
    ("infllmv2_topk_blocks", {}, (None, None, B, 1, 0, 0, 64, B, None), -1, "q is NULL"),
    ("infllmv2_topk_blocks", {}, (A, None, None, 1, 0, 0, 64, None, None), -1, "idx is NULL"),
    ("infllmv2_topk_blocks", {}, (A, None, None, 1, 300000, 0, 1 << 20, B, None), -2, "4096"),
    ("infllmv2_sparse_attn_prefill", {}, (A, 65, A, A, 64, 64, B, A, None, None), -1, "n_q"),
    ("infllmv2_sparse_attn_prefill", {}, (A, 64, A, A, 64, 64, None, A, None, None), -1, "idx is NULL"),
    ("infllmv2_sparse_attn_prefill", dict(top_k=1024), (A, 64, A, A, 64, 64, B, A, None, None), -2, "top_k"),
    ("infllmv2_sparse_attn_prefill", {}, (A, 64, A, A, 64, 64, B, A, A + 1, None), -1, "lse"),
    ("infllmv2_sparse_attn_decode", {}, (A, 1, A, A, 64, 64, B, None, A, None, A + 16, 1 << 30, None), -1, "workspace is not 256"),
    ("infllmv2_sparse_attn_decode", {}, (A, 1, A, A, 64, 64, B, None, A, None, 0x100000, 16, None), -3, "workspace"),
    ("infllmv2_sparse_attn_decode", {}, (A, 65, A, A, 128, 128, B, None, A, None, 0x100000, 1 << 30, None), -1, "64 query rows"),
    ("infllmv2_sparse_attn_decode", {}, (A, 2, A, A, 128, 128, B, A + 4, A, None, 0x100000, 1 << 30, None), -1, "tree_mask"),
    ("infllmv2_sparse_attn_decode_scores", {}, (A, A, A, 64, 64, None, None, B, None, 0x100000, 1 << 30, None), -1, "scores is NULL"),
    ("infllmv2_sparse_attn_decode_scores", {}, (A, A, A, 64, 64, A + 2, None, B, None, 0x100000, 1 << 30, None), -1, "scores"),
    ("infllmv2_sparse_attn_decode_scores", dict(top_k=65), (A, A, A, 64, 64, A, None, B, None, 0x100000, 1 << 30, None), -2, "top_k above 64"),
    ("infllmv2_sparse_attn_decode_scores", {}, (A, A, A, 1 << 20, 1 << 20, A, None, B, None, 0x100000, 1 << 40, None), -2, "4096"),
    ("infllmv2_sparse_attn_decode_scores", {}, (A, A, A, 64, 64, A, None, B, None, 0x100000, 16, None), -3, "workspace"),
    ("infllmv2_sparse_attn_prefill_backward", {}, (A, 64, A, A, 64, 64, B, A, None, A, A, A, A, 0x100000, 1 << 30, None), -1, "lse is NULL"),
    ("infllmv2_sparse_attn_prefill_backward", {}, (A, 64, A, A, 64, 64, B, A, B, None, A, A, A, 0x100000, 1 << 30, None), -1, "dout is NULL"),
    ("infllmv2_sparse_attn_prefill_backward", {}, (A, 64, A, A, 64, 64, B, A, B, A, A + 4, A, A, 0x100000, 1 << 30, None), -1, "dq"),
    ("infllmv2_sparse_attn_prefill_backward", {}, (A, 64, A, A, 64, 64, B, A, B, A, A, A, A, 0x100000, 16, None), -3, "workspace"),
    ("infllmv2_sparse_attn_prefill_backward", {}, (A, 65, A, A, 64, 64, B, A, B, A, A, A, A, 0x100000, 1 << 30, None), -1, "n_q"),
    ("infllmv2_dense_attn", {}, (A, 1, A, A, 64, 0, 1, B, None, None), -1, "kv_len"),
    ("infllmv2_dense_attn", {}, (A, 1, A, None, 64, 64, 1, B, None, None), -1, "v is NULL"),
    ("infllmv2_dense_attn", dict(softmax_scale=float("nan")), (A, 1, A, A, 64, 64, 1, B, None, None), -1, "finite"),
    ("infllmv2_append_kv", {}, (A, A, 1, A, A, 64, None, 64, None, None), -1, "exceeds kv_cap"),
    ("infllmv2_append_kv", {}, (A, A, -1, A, A, 64, None, 0, None, None), -1, "n_new"),
    ("infllmv2_append_kv", {}, (A, None, 1, A, A, 64, None, 0, None, None), -1, "v_new is NULL"),
    ("infllmv2_append_kv", {}, (A, A, 1, A, A, 64, A + 4, 0, None, None), -1, "kv_lens"),
    ("infllmv2_append_kv", {}, (A, A, 1, A, A, 64, None, 0, A + 2, None), -1, "kbar"),
    ("infllmv2_score_blocks_varlen", {}, (A, None, A, 64, A, None), -1, "kv_lens is NULL"),
    ("infllmv2_score_blocks_varlen", {}, (A, A, A, 0, A, None), -1, "kv_cap"),
    ("infllmv2_sparse_attn_decode_varlen", {}, (A, A, A, 64, None, 64, A, None, B, None, 0x100000, 1 << 30, None), -1, "kv_lens is NULL"),
    ("infllmv2_sparse_attn_decode_varlen", {}, (A, A, A, 64, A, 65, A, None, B, None, 0x100000, 1 << 30, None), -1, "exceeds kv_cap"),
    ("infllmv2_sparse_attn_decode_varlen", {}, (A, A, A, 64, A, 64, None, None, B, None, 0x100000, 1 << 30, None), -1, "scores is NULL"),
    ("infllmv2_sparse_attn_decode_varlen", dict(top_k=65), (A, A, A, 64, A, 64, A, None, B, None, 0x100000, 1 << 30, None), -2, "top_k above 64"),
    ("infllmv2_sparse_attn_decode_varlen", {}, (A, A, A, 64, A, 64, A, None, B, None, 0x100000, 16, None), -3, "workspace"),
    ("infllmv2_score_blocks_lse", {}, (A, 1, 0, 0, B, 64, A, None, 0, None), -1, "workspace is NULL"),
    ("infllmv2_score_blocks_lse", {}, (A, 1, 0, 0, B, 64, A, 0x100000, 16, None), -3, "workspace"),
    ("infllmv2_score_blocks_lse", {}, (A, 1, 640, 0, B, 64, A, 0x100000, 1 << 30, None), -1, "beyond kv_cap"),
    ("infllmv2_sliding_window_attn", {}, (A, 1, A, A, 64, 64, 0, B, None, None), -1, "window"),
    ("infllmv2_sliding_window_attn", {}, (A, 65, A, A, 64, 64, 16, B, None, None), -1, "n_q"),
    ("infllmv2_sliding_window_attn", {}, (A, 1, A, A, 64, 64, 16, None, None, None), -1, "out is NULL"),
]


@pytest.mark.parametrize("name,over,args,status,frag", CASES)
def test_rejected_before_any_hip_call(t, name, over, args, status, frag):
    cfg = None if over is None else cfg_ok(t, **over)
    rc, msg = call(t, name, cfg, *args)
    assert rc == status, msg
    assert frag in msg and name in msg


def test_empty_append_is_a_no_op_without_device_work(t):
    cfg = cfg_ok(t)
    rc, msg = call(t, "infllmv2_append_kv", cfg, A, A, 0, A, A, 64, None, 64, None, None)
    assert rc == 0, msg


def test_strerror(t):
    assert t.infllmv2_strerror(0) == "ok"
    assert t.infllmv2_strerror(-1) == "invalid argument"
    assert t.infllmv2_strerror(-2) == "unsupported"
    assert t.infllmv2_strerror(-3) == "workspace too small"
    assert t.infllmv2_strerror(-4) == "HIP error"
    assert t.infllmv2_strerror(7) == "unknown status"


def test_workspace_bytes(t):
    cfg = cfg_ok(t, batch=8, top_k=32)
    n1 = t.infllmv2_decode_workspace_bytes(cfg, 1, 131072)
    n16 = t.infllmv2_decode_workspace_bytes(cfg, 16, 131088)
    assert n1 > 0 and n16 > n1
    assert t.infllmv2_decode_workspace_bytes(cfg, 0, 10) == 0
    assert t.infllmv2_decode_workspace_bytes(cfg, 5, 3) == 0
    cfg = cfg_ok(t, top_k=16)
    b1 = t.infllmv2_prefill_backward_workspace_bytes(cfg, 32768, 32768)
    assert b1 > 0 and t.infllmv2_prefill_backward_workspace_bytes(cfg, 1024, 1024) < b1
    assert t.infllmv2_prefill_backward_workspace_bytes(cfg, 0, 10) == 0
    # head_dim 64 adds zero-padded bf16 copies (q, out, dout, k, v) and fp32 dq, dk, dv at width 128
    c64 = cfg_ok(t, head_dim=64)
    b64 = t.infllmv2_prefill_backward_workspace_bytes(c64, 1024, 1024)
    b128 = t.infllmv2_prefill_backward_workspace_bytes(cfg_ok(t), 1024, 1024)
    rq, rk = 32 * 1024, 8 * 1024   # query rows (heads x tokens), key rows
    assert b64 >= b128 + 128 * (3 * 2 * rq + 2 * 2 * rk + 4 * rq + 2 * 4 * rk)
    # variable lengths: room for the larger of K + 1 entries and a dense row below the threshold
    v1 = t.infllmv2_decode_varlen_workspace_bytes(cfg_ok(t, batch=8, top_k=32), 131072)
    assert v1 >= t.infllmv2_decode_workspace_bytes(cfg_ok(t, batch=8, top_k=32), 1, 131072) > 0
    vd = t.infllmv2_decode_varlen_workspace_bytes(cfg_ok(t, batch=8, top_k=4, dense_threshold=8192), 131072)
    assert vd > t.infllmv2_decode_workspace_bytes(cfg_ok(t, batch=8, top_k=4, dense_threshold=8192), 1, 131072)
    assert t.infllmv2_decode_varlen_workspace_bytes(cfg, 0) == 0
    assert t.infllmv2_score_lse_workspace_bytes(cfg, 1, 131072) > 2048 * 4
    assert t.infllmv2_score_lse_workspace_bytes(cfg, 0, 131072) == 0


def test_binding_raises_with_status(t):
    cfg = cfg_ok(t)
    with pytest.raises(t.InfLLMv2Error) as e:
        t.infllmv2_dense_attn(cfg, A, 1, A, None, 64, 64, 1, B, None, stream=0)
    assert e.value.status == -1 and "v is NULL" in e.value.message


def test_valid_call_without_gpu_reports_hip_error(t):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, msg = call(t, "infllmv2_pool_kernels", cfg_ok(t), A, 64, 64, 0, B, None)
    assert rc == -4 and "HIP error" in msg


# kv_cap need not be a multiple of 64: the tables hold nblk = ceil(kv_cap / 64) blocks and the
# kernels bound every read at kv_len, so such a cache is accepted and the call reaches the device
# check (here, without a GPU, a HIP error), never INVALID_ARGUMENT.
KV_CAP_RAGGED = [
    ("infllmv2_pool_kernels", (A, 100, 100, 0, B, None)),
    ("infllmv2_score_blocks", (A, 1, 99, 0, B, 100, A, None)),
    ("infllmv2_topk_blocks", (A, None, None, 1, 99, 0, 100, B, None)),
    ("infllmv2_sparse_attn_prefill", (A, 64, A, A, 100, 100, B, A, None, None)),
    ("infllmv2_sparse_attn_decode_scores", (A, A, A, 100, 100, A, None, B, None, 0x100000, 1 << 30, None)),
    ("infllmv2_dense_attn", (A, 1, A, A, 100, 100, 1, B, None, None)),
    ("infllmv2_score_blocks_varlen", (A, A, A, 100, A, None)),
]


@pytest.mark.parametrize("name,args", KV_CAP_RAGGED)
def test_kv_cap_not_multiple_of_64_is_accepted(t, name, args):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, msg = call(t, name, cfg_ok(t), *args)
    assert rc == -4 and "HIP error" in msg, msg


def test_fused_topk_accepts_4096_candidates_for_every_group_size(t):
    """One or two query heads per group with up to 4096 candidates fit the fused path (fewer tokens per
    workgroup): the call passes every argument check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    for hq, hkv in [(2, 2), (4, 2), (8, 2), (32, 8)]:
        cfg = cfg_ok(t, n_q_heads=hq, n_kv_heads=hkv, head_dim=64)
        rc, msg = call(t, "infllmv2_topk_blocks", cfg, None, A, B, 16, 64 * 4096, 0, 64 * 4097, A, None)
        assert rc == -4 and "HIP error" in msg, (hq, hkv, msg)


def test_noalloc_decode_rejects_scratch_above_its_maximum(t):
    """The allocation-free decode checks the workspace the shape needs against its static scratch
    (16 MiB) before any HIP call."""
    cfg = cfg_ok(t, batch=256, n_q_heads=256, n_kv_heads=64, top_k=64)
    need = t.infllmv2_decode_workspace_bytes(cfg, 1, 131072)
    assert need > 16 << 20
    rc, msg = call(t, "infllmv2_sparse_attn_decode_scores_noalloc", cfg, A, A, A, 131072, 131072, A, None, B,
                   None, None)
    assert rc == -2 and "static scratch" in msg, msg


def test_package_binds_every_export(t):
    """Each exported C function has a Python binding of the same name on the package."""
    for name in t.EXPORTS:
        assert callable(getattr(t, name)), name
