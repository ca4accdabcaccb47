"""The C ABI on the CPU: the library loads, exports every declared symbol,
plans batches, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from cross_model_attention_mf_amd import mapflow as mf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mapflow.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z_0-9]+)\s*\(", txt)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert set(decl) == set(mf.EXPORTS), decl


def test_library_exports_every_declared_symbol():
    L = mf.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.mf_version().decode().startswith("mapflow-mi355x")
    assert L.mf_status_string(3).decode() == "MF_ERR_CAPACITY"


def _c_layout(tmp_path):
    """Offsets and sizes of the header's structs as gcc lays them out."""
    import subprocess
    fields = {
        "mf_plan_info": [f for f, _ in mf.PlanInfo._fields_],
        "mf_batch": [f for f, _ in mf.BatchC._fields_],
        "mf_sender_desc": [f for f, _ in mf.SenderDesc._fields_],
        "mf_receiver_desc": [f for f, _ in mf.ReceiverDesc._fields_],
        "mf_map_cache_desc": [f for f, _ in mf.MapCacheDesc._fields_],
        "mf_map_cache_stats": [f for f, _ in mf.MapCacheStats._fields_],
        "mf_headmix_desc": [f for f, _ in mf.HeadmixDesc._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mapflow.h"', 'int main(void) {']
    for st, fs in fields.items():
        lines.append(f'printf("{st} sizeof %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    return {tuple(ln.split()[:2]): int(ln.split()[2]) for ln in out.splitlines()}


def test_struct_layouts_match_header(tmp_path):
    c = _c_layout(tmp_path)
    for name, cls in [("mf_plan_info", mf.PlanInfo), ("mf_batch", mf.BatchC),
                      ("mf_sender_desc", mf.SenderDesc), ("mf_receiver_desc", mf.ReceiverDesc),
                      ("mf_map_cache_desc", mf.MapCacheDesc), ("mf_map_cache_stats", mf.MapCacheStats),
                      ("mf_headmix_desc", mf.HeadmixDesc)]:
        assert c[(name, "sizeof")] == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert c[(name, f)] == getattr(cls, f).offset, (name, f)


def test_plan_layout():
    cu_q = [0, 100, 164, 164, 400]
    cu_k = [0, 228, 292, 300, 936]
    p0 = [128, 0, 0, 384]
    info, plan = mf.plan(cu_q, cu_k, p0, 64)
    assert info.total_rowblocks == 2 + 1 + 0 + 4
    assert info.max_colblocks == (636 + 63) // 64
    assert info.total_q == 400 and info.total_k == 936 and info.max_k_len == 636
    assert list(plan[:5]) == [0, 2, 3, 3, 7]
    assert list(plan[5:]) == [0, 0, 1, 3, 3, 3, 3]


@pytest.mark.parametrize("args,status", [
    (([0, 10], [0, 5], None, 64), mf.MF_ERR_INVALID),          # keys do not cover queries
    (([0, 10], [0, 40], [30], 64), mf.MF_ERR_UNSUPPORTED),     # chunk not on a block edge
    (([0, 10], [0, 10], None, 48), mf.MF_ERR_UNSUPPORTED),     # unsupported B
    (([0, 10, 5], [0, 10, 20], None, 64), mf.MF_ERR_INVALID),  # negative length
    (([1, 10], [0, 10], None, 64), mf.MF_ERR_INVALID),         # offsets must start at 0
    (([0, 10], [0, 50000], None, 64), mf.MF_ERR_UNSUPPORTED),  # longer than MF_MAX_KEYS
])
def test_plan_errors(args, status):
    with pytest.raises(mf.MapflowError) as e:
        mf.plan(*args)
    assert e.value.status == status


def _host_batch(cu_q, cu_k, q_pos0, B):
    """A batch whose device pointers are fake: only for calls that must fail
    validation (or do nothing) before touching the GPU."""
    info, _ = mf.plan(cu_q, cu_k, q_pos0, B)
    b = mf.BatchC(info, 16, 16, None, 16)
    return b


def _sender(**kw):
    base = dict(dtype=mf.MF_BF16, num_layers=1, H_s=4, H_kv_s=4, d=128, B=64, sm_scale=0.0,
                layer_stride_q=0, layer_stride_k=0)
    base.update(kw)
    return mf.SenderDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=48), mf.MF_ERR_UNSUPPORTED),
    (dict(d=96), mf.MF_ERR_UNSUPPORTED),
    (dict(H_s=65, H_kv_s=65), mf.MF_ERR_UNSUPPORTED),
    (dict(H_kv_s=3), mf.MF_ERR_INVALID),
    (dict(dtype=7), mf.MF_ERR_INVALID),
    (dict(num_layers=-1), mf.MF_ERR_INVALID),
    (dict(sm_scale=float("nan")), mf.MF_ERR_INVALID),
    (dict(num_layers=2, layer_stride_q=5, layer_stride_k=5), mf.MF_ERR_INVALID),
])
def test_block_stats_validation(kw, status):
    b = _host_batch([0, 256], [0, 256], None, kw.get("B", 64) if kw.get("B", 64) in (32, 64, 128) else 64)
    d = _sender(**kw)
    st = mf.lib().mf_block_stats(ctypes.byref(d), ctypes.byref(b), 16, 16, 16, 16, None, 0, None)
    assert st == status, mf.lib().mf_last_error_message()
    assert mf.lib().mf_last_error_message().decode()


def test_block_mismatch_between_plan_and_desc():
    b = _host_batch([0, 256], [0, 256], None, 32)
    d = _sender(B=64)
    assert mf.lib().mf_block_stats(ctypes.byref(d), ctypes.byref(b), 16, 16, 16, 16, None, 0, None) == mf.MF_ERR_INVALID


def test_empty_batch_is_a_noop():
    b = _host_batch([0], [0], None, 64)
    d = _sender()
    assert mf.lib().mf_block_stats(ctypes.byref(d), ctypes.byref(b), None, None, None, None, None, 0, None) == mf.MF_OK


@pytest.mark.parametrize("tau", [0.0, -0.5, 1.5, float("nan")])
def test_compress_rejects_tau(tau):
    b = _host_batch([0, 256], [0, 256], None, 64)
    d = _sender()
    nnz = ctypes.c_int64(0)
    st = mf.lib().mf_compress_blocks(ctypes.byref(d), ctypes.byref(b), 16, 16, 16, 16, tau, 16, 16, 16,
                                     10, ctypes.byref(nnz), 16, 1 << 20, None)
    assert st == mf.MF_ERR_INVALID


def test_compress_workspace_checks():
    b = _host_batch([0, 256], [0, 256], None, 64)
    d = _sender()
    need = mf.lib().mf_compress_workspace_size(ctypes.byref(d), ctypes.byref(b))
    rows = 1 * 4 * 4
    assert need >= rows * 4 + rows * 1 * 4
    st = mf.lib().mf_compress_blocks(ctypes.byref(d), ctypes.byref(b), 16, 16, 16, 16, 0.9, 16, 16, 16,
                                     10, None, 16, need - 1, None)
    assert st == mf.MF_ERR_WORKSPACE
    st = mf.lib().mf_compress_blocks(ctypes.byref(d), ctypes.byref(b), 16, 16, 16, 16, 0.9, 16, 16, 16,
                                     -1, None, 16, need, None)
    assert st == mf.MF_ERR_INVALID


def _receiver(layer_map, **kw):
    lm = np.asarray(layer_map, dtype=np.int32)
    base = dict(dtype=mf.MF_BF16, num_layers=len(layer_map), sender_layers=2,
                layer_map=lm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), H_s=4, H_r=3, H_kv_r=3,
                d=128, B=64, layer_stride_v=1 << 30, layer_stride_o=1 << 30, block_table=None,
                page_size=0, max_pages=0, num_pages=0, csr_capacity=16)
    base.update(kw)
    r = mf.ReceiverDesc(**base)
    r._keep = lm
    return r


@pytest.mark.parametrize("layer_map,kw,status", [
    ([0, 2], {}, mf.MF_ERR_INVALID),                       # sender layer out of range
    ([0, -1], {}, mf.MF_ERR_INVALID),
    ([0], dict(H_kv_r=2), mf.MF_ERR_INVALID),               # kv heads do not divide
    ([0], dict(H_s=0), mf.MF_ERR_UNSUPPORTED),
    ([0], dict(block_table=16, page_size=0, max_pages=4, num_pages=4), mf.MF_ERR_INVALID),
    ([0], dict(block_table=16, page_size=16, max_pages=1, num_pages=4), mf.MF_ERR_INVALID),  # table too short
])
def test_mapped_validation(layer_map, kw, status):
    b = _host_batch([0, 256], [0, 256], None, 64)
    r = _receiver(layer_map, **kw)
    st = mf.lib().mf_mapped_attn_v(ctypes.byref(r), ctypes.byref(b), 16, 16, 16, 16, 16, 16, None)
    assert st == status, mf.lib().mf_last_error_message()


@pytest.mark.parametrize("layer_map,kw,status", [
    ([0, 2], {}, mf.MF_ERR_INVALID),
    ([0], dict(H_kv_r=2), mf.MF_ERR_INVALID),
    ([0], dict(H_s=0), mf.MF_ERR_UNSUPPORTED),
    ([0], dict(block_table=16, page_size=16, max_pages=1, num_pages=4), mf.MF_ERR_INVALID),
])
def test_mapped_split_validation(layer_map, kw, status):
    """The split entry point validates its receiver as mf_mapped_attn_v does,
    before looking at the workspace."""
    b = _host_batch([0, 256], [0, 256], None, 64)
    r = _receiver(layer_map, **kw)
    st = mf.lib().mf_mapped_attn_v_split(ctypes.byref(r), ctypes.byref(b), 16, 16, 16, 16, 16, 16, None, 0, None)
    assert st == status, mf.lib().mf_last_error_message()


def test_mapped_split_workspace_size_of_invalid_arguments_is_zero():
    b = _host_batch([0, 256], [0, 256], None, 64)
    lib = mf.lib()
    assert lib.mf_mapped_split_workspace_size(None, ctypes.byref(b)) == 0
    assert lib.mf_mapped_split_workspace_size(ctypes.byref(_receiver([0])), None) == 0
    assert lib.mf_mapped_split_workspace_size(ctypes.byref(_receiver([0], num_layers=-1)), ctypes.byref(b)) == 0


def test_mapped_split_empty_batch_is_a_noop():
    b = _host_batch([0, 0], [0, 0], None, 64)
    r = _receiver([0])
    assert mf.lib().mf_mapped_attn_v_split(ctypes.byref(r), ctypes.byref(b), None, None, None, None, None, None,
                                           None, 0, None) == mf.MF_OK


def test_mfma_probe_rejects_bad_arguments():
    lib = mf.lib()
    assert lib.mf_mfma_probe(None, 4, 10, 0, None) == mf.MF_ERR_INVALID
    assert lib.mf_mfma_probe(16, 0, 10, 0, None) == mf.MF_ERR_INVALID
    assert lib.mf_mfma_probe(16, 4, 0, 1, None) == mf.MF_ERR_INVALID


def _multi(descs, ptrs=16):
    n = len(descs)
    dp = (ctypes.POINTER(mf.ReceiverDesc) * max(n, 1))(*[ctypes.pointer(d) for d in descs])
    arr = (ctypes.c_void_p * max(n, 1))(*([ptrs] * max(n, 1)))
    return dp, arr


@pytest.mark.parametrize("case", ["null", "zero", "too_many", "shared_field", "layer_map", "per_receiver"])
def test_mapped_multi_validation(case):
    b = _host_batch([0, 256], [0, 256], None, 64)
    r0 = _receiver([0, 1])
    descs = [r0, _receiver([0, 1], H_r=8, H_kv_r=2)]
    n = len(descs)
    if case == "shared_field":
        descs[1] = _receiver([0, 1], H_s=5)
    elif case == "layer_map":
        descs[1] = _receiver([1, 0])
    elif case == "per_receiver":
        descs[1] = _receiver([0, 1], H_kv_r=5)            # kv heads do not divide H_r
    elif case == "too_many":
        descs = [r0] * (mf.MF_MAX_RECEIVERS + 1)
        n = len(descs)
    elif case == "zero":
        n = 0
    dp, arr = _multi(descs)
    if case == "null":
        st = mf.lib().mf_mapped_attn_v_multi(dp, n, ctypes.byref(b), 16, 16, 16, None, arr, arr, None)
    else:
        st = mf.lib().mf_mapped_attn_v_multi(dp, n, ctypes.byref(b), 16, 16, 16, arr, arr, arr, None)
    assert st == mf.MF_ERR_INVALID, mf.lib().mf_last_error_message()


def test_mapped_multi_empty_batch_is_a_noop():
    b = _host_batch([0, 0], [0, 0], None, 64)
    descs = [_receiver([0]), _receiver([0], H_r=8, H_kv_r=8)]
    dp, arr = _multi(descs, ptrs=None)
    assert mf.lib().mf_mapped_attn_v_multi(dp, 2, ctypes.byref(b), None, None, None, arr, arr, arr, None) == mf.MF_OK


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mf, "_lib", None)
    monkeypatch.setattr(mf, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mf.lib()


# ---- prefix cache of compressed maps: host-side behaviour (no device work)

def test_prefix_block_hashes_match_oracle_chain():
    from oracle import prefix_hash_oracle as ph
    rng = np.random.default_rng(7)
    toks = rng.integers(-2**31, 2**31, size=1000, dtype=np.int64).astype(np.int32)
    for B, parent in [(64, 0), (32, 0x0123456789ABCDEF), (7, 5)]:
        got = mf.prefix_block_hashes(toks, B, parent)
        want = ph.prefix_block_keys(toks.tolist(), B, parent)
        assert len(got) == len(toks) // B
        assert [int(x) for x in got] == want
    # keys chain: a continuation from the last key of a prefix equals the tail
    # of the whole sequence's keys
    full = mf.prefix_block_hashes(toks[:640], 64)
    tail = mf.prefix_block_hashes(toks[320:640], 64, int(full[4]))
    assert list(tail) == list(full[5:])
    assert len(mf.prefix_block_hashes(toks[:63], 64)) == 0
    assert mf.lib().mf_prefix_block_hashes(None, 10, 64, 0, None) == -1


def test_map_cache_host_paths():
    # a fake 256-byte aligned "device" address: create, lookup and release
    # touch only the host index
    d = mf.MapCacheDesc(mf.MF_BF16, 2, 4, 64)
    h = ctypes.c_void_p()
    L = mf.lib()
    assert L.mf_map_cache_create(ctypes.byref(d), 1 << 20, 1 << 20, ctypes.byref(h)) == mf.MF_OK
    try:
        keys = (ctypes.c_uint64 * 3)(1, 2, 3)
        assert L.mf_map_cache_lookup(h, keys, 3) == 0
        L.mf_map_cache_release(h, keys, 0)
        st = mf.MapCacheStats()
        assert L.mf_map_cache_get_stats(h, ctypes.byref(st)) == mf.MF_OK
        assert st.blocks_missed == 3 and st.entries == 0 and st.bytes_capacity > 0
        # splice with nothing cached refuses a cached prefix it does not hold
        nnz = ctypes.c_int64()
        rp = (ctypes.c_int32 * 2)(0, 0)
        assert L.mf_map_cache_splice(h, keys, 1, 2, rp, 1, 0, None, None, 16, None, None, 0,
                                     ctypes.byref(nnz), None) == mf.MF_ERR_INVALID
        # insert argument checks come before any copy
        assert L.mf_map_cache_insert(h, keys, 0, rp, 1, 0, None, None, None) == mf.MF_ERR_INVALID
        assert L.mf_map_cache_insert(h, keys, 2, rp, 1, 0, None, None, None) == mf.MF_ERR_INVALID
    finally:
        L.mf_map_cache_destroy(h)
    bad = mf.MapCacheDesc(mf.MF_BF16, 0, 4, 64)
    assert L.mf_map_cache_create(ctypes.byref(bad), 1 << 20, 1 << 20, ctypes.byref(h)) == mf.MF_ERR_INVALID
    assert L.mf_map_cache_create(ctypes.byref(d), (1 << 20) + 16, 1 << 20, ctypes.byref(h)) == mf.MF_ERR_INVALID
    assert L.mf_map_cache_create(ctypes.byref(d), 1 << 20, 512, ctypes.byref(h)) == mf.MF_ERR_CAPACITY


# ---- head-mix fit: argument checks come before any launch

def test_headmix_validation_paths():
    L = mf.lib()
    info, plan = mf.plan([0, 200], [0, 200], None, 64)
    fake = 1 << 20   # never dereferenced: every call below fails validation or has no work
    bc = mf.BatchC(info, fake, fake, None, fake)
    good = mf.headmix_desc(torch.bfloat16, 64, [1, 0], 2, 8, 6, 100, 100)
    need = L.mf_headmix_workspace_size(ctypes.byref(good), ctypes.byref(bc))
    assert need == -(-2 * info.total_rowblocks * (8 + 6) * 8 * 8 // 256) * 256   # fp64 partials, 256-byte rounded

    def gram(desc, ws=fake, ws_bytes=None, gram_ptr=fake):
        return L.mf_headmix_gram(ctypes.byref(desc), ctypes.byref(bc), fake, fake, fake, fake, fake, fake,
                                 gram_ptr, fake, ws, need if ws_bytes is None else ws_bytes, None)
    assert gram(mf.headmix_desc(torch.bfloat16, 48, [0], 1, 8, 6, 1, 1)) == mf.MF_ERR_UNSUPPORTED
    assert gram(mf.headmix_desc(torch.bfloat16, 64, [0], 1, 65, 6, 1, 1)) == mf.MF_ERR_UNSUPPORTED
    assert gram(mf.headmix_desc(torch.bfloat16, 64, [2], 2, 8, 6, 1, 1)) == mf.MF_ERR_INVALID
    assert gram(mf.headmix_desc(torch.bfloat16, 64, [0], 1, 8, 6, -1, 1)) == mf.MF_ERR_INVALID
    assert gram(mf.headmix_desc(torch.bfloat16, 32, [0], 1, 8, 6, 1, 1)) == mf.MF_ERR_INVALID  # batch planned for 64
    assert gram(good, ws_bytes=need - 1) == mf.MF_ERR_WORKSPACE
    assert L.mf_headmix_gram(ctypes.byref(good), ctypes.byref(bc), fake, fake, fake + 8, fake, fake, fake,
                             fake, fake, fake, need, None) == mf.MF_ERR_INVALID   # misaligned values
    assert gram(good, gram_ptr=None) == mf.MF_ERR_INVALID
    assert "gram" in L.mf_last_error_message().decode()
    # no layers: nothing to do
    assert gram(mf.headmix_desc(torch.bfloat16, 64, [], 2, 8, 6, 1, 1), ws=None, ws_bytes=0) == mf.MF_OK

    def solve(desc, lam=0.0, W=fake):
        return L.mf_headmix_solve(ctypes.byref(desc), fake, fake, lam, W, None, None)
    assert solve(good, lam=-1.0) == mf.MF_ERR_INVALID
    assert solve(good, lam=float("inf")) == mf.MF_ERR_INVALID
    assert solve(good, lam=float("nan")) == mf.MF_ERR_INVALID
    assert solve(good, W=None) == mf.MF_ERR_INVALID
    assert solve(mf.headmix_desc(torch.bfloat16, 64, [0], 1, 0, 6, 1, 1)) == mf.MF_ERR_UNSUPPORTED


def test_layer_group_pipeline_rejects_bad_group_counts():
    import torch
    from cross_model_attention_mf_amd import pipeline
    q = torch.zeros((4, 8, 2, 64), dtype=torch.bfloat16)
    for g in (0, 5):
        with pytest.raises(ValueError):
            pipeline.LayerGroupPipeline(None, q, q, q, None, None, 64, 0.9, 2, g)


def test_force_portable_hook_round_trip():
    L = mf.lib()
    assert L.mf_debug_force_portable(0) == 0
    with mf.force_portable("stats", "mapped"):
        # unknown bits are dropped; the previous mask comes back
        assert L.mf_debug_force_portable(0xFFFFFFFF) == 0x9
        assert L.mf_debug_force_portable(0x9) == 0xF
    assert L.mf_debug_force_portable(0) == 0
