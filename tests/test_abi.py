"""The C ABI on the host (no GPU): the library loads, exports every entry point
that include/qsa.h declares, rejects malformed calls before any launch, sizes
workspaces and picks the documented route for each workload."""
import ctypes
import os
import re

import pytest
import torch

from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000   # never dereferenced: every case below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "qsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qsa_\w+)\s*\(", text, re.M)))


def cfg_for(w, **kw):
    args = dict(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads,
                num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, rotary_dim=w.rotary_dim,
                rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                max_seq_len=(w.ragged[1] if w.ragged else w.prior) + w.q_len,
                q_norm_w=FAKE, k_norm_w=FAKE)
    args.update(kw)
    return binding.make_cfg(**args)


def test_library_exports_every_declared_entry_point():
    lib = binding.load()
    declared = header_functions()
    assert set(binding.EXPORTS) <= set(declared)
    assert len(declared) >= 5
    for name in declared:
        assert hasattr(lib, name), name


def test_library_is_gfx950_code_object():
    data = open(binding.library_path(), "rb").read()
    assert b"gfx950" in data


@pytest.mark.parametrize("name,route", [("tiny_f32", "f32_rows"), ("decode_4b", "fused_splitk"),
                                        ("verify_24x2", "fused_splitk"), ("ragged_4b", "fused_splitk"),
                                        ("prefill_4b", "prepared_tiles")])
def test_route_per_workload(name, route):
    plan = binding.describe_plan(cfg_for(WORKLOADS[name]))
    assert f"route={route}" in plan
    fields = dict(kv.split("=") for kv in plan.split())
    assert int(fields["workspace"]) == binding.workspace_size(cfg_for(WORKLOADS[name]))


@pytest.mark.parametrize("geo,route", [
    (dict(head_dim=256, rotary_dim=64, q_len=1, num_q_heads=16, num_kv_heads=4), "fused_splitk"),
    (dict(head_dim=256, rotary_dim=32, q_len=4, num_q_heads=24, num_kv_heads=2), "fused_splitk"),   # 48 rows
    (dict(head_dim=64, rotary_dim=8, q_len=3, num_q_heads=8, num_kv_heads=2), "fused_splitk"),
    (dict(head_dim=128, rotary_dim=0, q_len=16, num_q_heads=3, num_kv_heads=1), "fused_splitk"),
    (dict(head_dim=256, rotary_dim=16, q_len=1, num_q_heads=16, num_kv_heads=4), "prepared_tiles"),  # r/2 % 16
    (dict(head_dim=128, rotary_dim=24, q_len=1, num_q_heads=4, num_kv_heads=1), "prepared_tiles"),   # r/2 % 8
    (dict(head_dim=256, rotary_dim=64, q_len=7, num_q_heads=7, num_kv_heads=1), "prepared_tiles"),   # 49 rows
    (dict(head_dim=256, rotary_dim=128, q_len=16, num_q_heads=2, num_kv_heads=1), "prepared_tiles"),  # L r/2 = 1024
    (dict(head_dim=256, rotary_dim=64, q_len=17, num_q_heads=1, num_kv_heads=1), "prepared_tiles"),   # L > 16
])
def test_short_query_route_limits(geo, route):
    """The short-query kernel takes at most 48 query rows and 16 new rows per
    sequence, tabulates at most 512 (cos, sin) pairs, and rotates by whole
    lanes (r/2 a multiple of head_dim/16); anything else takes the tile route."""
    w = Workload("limits", batch=2, rope_theta=1e7, dtype="bf16", prior=100, seed=1, **geo)
    assert f"route={route}" in binding.describe_plan(cfg_for(w))


def test_plan_covers_max_seq_len_and_forced_splits():
    w = WORKLOADS["decode_4b"]
    for k in (1, 2, 7, 65):
        f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(w, force_splits=k)).split())
        chunks, ck = int(f["chunks"]), int(f["chunk_keys"])
        # chunks of chunk_keys keys, the last one also taking the remainder
        assert chunks * ck <= 4097 < (chunks + 1) * ck
        assert k <= chunks <= k + 1


def test_default_plans_fill_one_round_for_short_work():
    f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(WORKLOADS["decode_4b"])).split())
    assert int(f["workgroups"]) == 256
    f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(WORKLOADS["verify_24x2"])).split())
    assert int(f["workgroups"]) == 256


def test_split_merge_placement_per_route():
    """Calls whose grid splits keys merge the partials in a second kernel
    (plan field merge=kernel); unsplit calls launch no merge."""
    for name in ("decode_4b", "verify_24x2", "ragged_4b", "prefill_4b"):
        f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(WORKLOADS[name])).split())
        assert f["merge"] == "kernel" and int(f["chunks"]) > 1, name
    f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(WORKLOADS["tiny_f32"])).split())
    assert f["merge"] == "none"
    one = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(WORKLOADS["decode_4b"], force_splits=1)).split())
    assert one["merge"] == "none"


def test_tile_route_plan_fills_the_chip_with_equal_chunks():
    """Prefill: 256-row tiles of 512 threads, and just enough equal key chunks
    per tile (none shorter than 1024 keys) that the grid gives every CU one
    workgroup; a forced count is capped by the 32-key minimum."""
    w = WORKLOADS["prefill_4b"]
    f = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(w)).split())
    rows = w.q_len * w.num_q_heads // w.num_kv_heads
    assert int(f["rows"]) == 256 and int(f["threads"]) == 512
    assert int(f["tiles"]) == -(-rows // 256)
    slots = w.batch * w.num_kv_heads * int(f["tiles"])
    assert int(f["chunks"]) == -(-256 // slots) and int(f["chunk_keys"]) == 1024
    assert int(f["workgroups"]) == slots * int(f["chunks"]) == 256
    for k in (1, 3, 5000):
        g = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(w, force_splits=k)).split())
        assert int(g["chunks"]) == min(k, 32768 // 32) and int(g["chunk_keys"]) == 32
    # two sequences' tiles already fill the chip: one chunk each
    w2 = Workload("prefill_b2", batch=2, q_len=2048, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
                  rope_theta=1e7, dtype="bf16", prior=30720, seed=1)
    g = dict(kv.split("=") for kv in binding.describe_plan(cfg_for(w2)).split())
    assert int(g["chunks"]) == 1 and int(g["workgroups"]) == 256


@pytest.mark.parametrize("bad,code", [
    (dict(num_q_heads=6, num_kv_heads=4), binding.QSA_ERR_INVALID),
    (dict(rotary_dim=63), binding.QSA_ERR_INVALID),
    (dict(rotary_dim=258), binding.QSA_ERR_INVALID),
    (dict(head_dim=96, rotary_dim=32), binding.QSA_ERR_UNSUPPORTED),
    (dict(dtype=7), binding.QSA_ERR_UNSUPPORTED),
    (dict(max_seq_len=0), binding.QSA_ERR_INVALID),
    (dict(q_len=0), binding.QSA_ERR_INVALID),
    (dict(rope_theta=-1.0), binding.QSA_ERR_INVALID),
    (dict(rms_eps=float("nan")), binding.QSA_ERR_INVALID),
    (dict(q_norm_w=None), binding.QSA_ERR_INVALID),
    (dict(force_splits=-2), binding.QSA_ERR_INVALID),
])
def test_invalid_configurations_are_rejected(bad, code):
    cfg = cfg_for(WORKLOADS["decode_4b"], **bad)
    lib = binding.load()
    assert lib.qsa_workspace_size(ctypes.byref(cfg)) == 0
    assert binding.last_error() != ""
    kv = binding.KVCache(FAKE, FAKE + (1 << 30), FAKE, None, 8192)
    rc = lib.qsa_gated_attention(FAKE, None, None, ctypes.byref(kv), FAKE, FAKE, ctypes.byref(cfg),
                                 FAKE + (2 << 30))
    assert rc == code, binding.last_error()


def test_argument_errors_before_launch():
    w = WORKLOADS["decode_4b"]
    lib = binding.load()
    kv = binding.KVCache(FAKE, FAKE + (1 << 30), FAKE, None, 8192)
    need = binding.workspace_size(cfg_for(w))
    small = cfg_for(w)
    small.workspace, small.workspace_bytes = FAKE + (3 << 30), need - 1
    out = FAKE + (2 << 30)
    call = lambda q, k, v, kvd, sl, pos, c, o: lib.qsa_gated_attention(
        q, k, v, ctypes.byref(kvd) if kvd is not None else None, sl, pos, ctypes.byref(c), o)
    assert call(FAKE, FAKE, FAKE, kv, FAKE, FAKE, small, out) == binding.QSA_ERR_WORKSPACE
    assert "workspace" in binding.last_error()
    assert call(FAKE, FAKE, None, kv, FAKE, FAKE, small, out) == binding.QSA_ERR_INVALID
    assert call(None, FAKE, FAKE, kv, FAKE, FAKE, small, out) == binding.QSA_ERR_INVALID
    assert call(FAKE, FAKE, FAKE, None, FAKE, FAKE, small, out) == binding.QSA_ERR_INVALID
    same = binding.KVCache(FAKE, FAKE, FAKE, None, 8192)
    assert call(FAKE, FAKE, FAKE, same, FAKE, FAKE, small, out) == binding.QSA_ERR_INVALID
    # output aliasing the query input
    assert call(FAKE, FAKE, FAKE, kv, FAKE, FAKE, small, FAKE + 64) == binding.QSA_ERR_INVALID
    assert "alias" in binding.last_error()
    assert lib.qsa_append_kv(None, FAKE, ctypes.byref(kv), FAKE, FAKE, ctypes.byref(small)) == \
        binding.QSA_ERR_INVALID


def test_noalloc_entry_point_checks_before_any_launch():
    """The allocation-free entry point validates like qsa_gated_attention and
    rejects a plan that needs more than its fixed scratch (a 12288-row prefill
    chunk of the 4B geometry needs 96 MiB of prepared queries) with
    QSA_ERR_WORKSPACE, before touching a device."""
    lib = binding.load()
    kv = binding.KVCache(FAKE, FAKE + (1 << 30), FAKE, None, 1 << 20)
    out = FAKE + (2 << 30)
    big = cfg_for(WORKLOADS["prefill_4b"].with_(q_len=12288))
    assert binding.workspace_size(big) > binding.NOALLOC_SCRATCH_BYTES
    rc = lib.qsa_gated_attention_noalloc(FAKE, FAKE, FAKE, ctypes.byref(kv), FAKE, FAKE, ctypes.byref(big), out)
    assert rc == binding.QSA_ERR_WORKSPACE
    assert "scratch" in binding.last_error()
    bad = cfg_for(WORKLOADS["decode_4b"], rotary_dim=63)
    rc = lib.qsa_gated_attention_noalloc(FAKE, FAKE, FAKE, ctypes.byref(kv), FAKE, FAKE, ctypes.byref(bad), out)
    assert rc == binding.QSA_ERR_INVALID
    for name in ("decode_4b", "verify_24x2", "ragged_4b", "prefill_4b"):
        assert binding.workspace_size(cfg_for(WORKLOADS[name])) <= binding.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "qsa.h")).read()
    m = re.search(r"#define QSA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES


def test_projection_arguments_checked_before_launch():
    lib = binding.load()
    ok = cfg_for(WORKLOADS["decode_4b"])
    call = lambda c, hidden, *ptrs: lib.qsa_qkv_proj(*ptrs[:2], hidden, ctypes.byref(c), *ptrs[2:])
    q, k, v, x, w = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)
    assert call(ok, 2560, x, w, q, k, None) == binding.QSA_ERR_INVALID
    assert call(ok, 2500, x, w, q, k, v) == binding.QSA_ERR_UNSUPPORTED          # hidden % 256
    assert call(cfg_for(WORKLOADS["decode_4b"], batch=65), 2560, x, w, q, k, v) == binding.QSA_ERR_UNSUPPORTED
    assert call(cfg_for(WORKLOADS["tiny_f32"]), 2560, x, w, q, k, v) == binding.QSA_ERR_UNSUPPORTED   # fp32
    assert call(ok, 2560, x, w, q, q + 64, v) == binding.QSA_ERR_INVALID          # outputs overlap
    assert call(ok, 2560, x, w, x, k, v) == binding.QSA_ERR_INVALID               # output aliases x
    assert lib.qsa_o_proj(x, w, 2560, ctypes.byref(ok), x + 8) == binding.QSA_ERR_INVALID
    assert lib.qsa_o_proj(x, None, 2560, ctypes.byref(ok), q) == binding.QSA_ERR_INVALID


def test_paged_cache_descriptor_checked_before_launch():
    lib = binding.load()
    w = WORKLOADS["decode_4b"]
    c = cfg_for(w)
    c.workspace, c.workspace_bytes = FAKE + (3 << 30), binding.workspace_size(cfg_for(w))
    out = FAKE + (2 << 30)

    def call(kv, cfg=c):
        return lib.qsa_gated_attention(FAKE, FAKE, FAKE, ctypes.byref(kv), FAKE, FAKE, ctypes.byref(cfg), out)

    for bs, rows, mb in ((48, 4800, 8), (32, 4096, 8), (96, 4800, 8), (64, 4100, 8), (64, 4096, 0)):
        kv = binding.KVCache(FAKE, FAKE + (1 << 30), None, None, rows, FAKE + (4 << 30), bs, mb)
        assert call(kv) == binding.QSA_ERR_INVALID, (bs, rows, mb)
    # a contiguous cache needs seq_offset
    assert call(binding.KVCache(FAKE, FAKE + (1 << 30), None, None, 8192)) == binding.QSA_ERR_INVALID
    # the tile route takes no paged cache
    p = cfg_for(WORKLOADS["prefill_4b"])
    p.workspace, p.workspace_bytes = FAKE + (3 << 30), binding.workspace_size(cfg_for(WORKLOADS["prefill_4b"]))
    kv = binding.KVCache(FAKE, FAKE + (1 << 30), None, None, 1 << 16, FAKE + (4 << 30), 64, 600)
    assert call(kv, p) == binding.QSA_ERR_UNSUPPORTED
    # chunks longer than 128 blocks
    f = cfg_for(w, force_splits=1)
    f.workspace, f.workspace_bytes = FAKE + (3 << 30), binding.workspace_size(cfg_for(w, force_splits=1))
    kv = binding.KVCache(FAKE, FAKE + (1 << 30), None, None, 1 << 16, FAKE + (4 << 30), 64, 80)
    assert call(kv, f) == binding.QSA_ERR_UNSUPPORTED
    assert "128 blocks" in binding.last_error()


def test_gdn_arguments_checked_before_launch():
    lib = binding.load()
    ptrs = [FAKE + (i << 30) for i in range(11)]

    def call(cfg, p=ptrs):
        return lib.qsa_gdn_decode(*p, ctypes.byref(cfg))

    def cfg(**kw):
        a = dict(batch=4, num_k_heads=16, num_v_heads=32, k_head_dim=128, v_head_dim=128, conv_kernel=4,
                 stream=None)
        a.update(kw)
        return binding.make_gdn_cfg(**a)

    assert call(cfg(num_v_heads=24)) == binding.QSA_ERR_INVALID                  # not a multiple of Hk
    assert call(cfg(num_v_heads=48)) == binding.QSA_ERR_UNSUPPORTED              # Hv / Hk = 3
    assert call(cfg(k_head_dim=64)) == binding.QSA_ERR_UNSUPPORTED
    assert call(cfg(conv_kernel=5)) == binding.QSA_ERR_UNSUPPORTED
    assert call(cfg(batch=-1)) == binding.QSA_ERR_INVALID
    assert call(cfg(), ptrs[:10] + [None]) == binding.QSA_ERR_INVALID            # y missing
    assert call(cfg(), ptrs[:10] + [ptrs[0] + 64]) == binding.QSA_ERR_INVALID    # y aliases qkv
    assert call(cfg(), ptrs[:9] + [ptrs[8] + 16, ptrs[10]]) == binding.QSA_ERR_INVALID   # states overlap
    assert call(cfg(), ptrs[:10] + [ptrs[10] + 8]) == binding.QSA_ERR_INVALID    # misaligned
    assert "aligned" in binding.last_error()


def test_workspace_scales_with_chunks():
    w = WORKLOADS["decode_4b"]
    one = binding.workspace_size(cfg_for(w, force_splits=1))
    many = binding.workspace_size(cfg_for(w, force_splits=32))
    assert many > one >= 256


def test_ctypes_structs_match_the_header_layout(tmp_path):
    """Every field of the ctypes mirrors sits at the offset a C compiler gives it."""
    structs = {"qsa_cfg": binding.Cfg, "qsa_kv_cache": binding.KVCache, "qsa_gdn_cfg": binding.GdnCfg}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "qsa.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
