"""C-ABI boundary checks that need no GPU: exports, struct layout, admission, split policy."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from verify_attention_e4m3_amd import attention as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 11, names
    lib = A.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(A.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(names)          # nothing else leaks out of the library


def test_struct_layout_matches_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "attn.h"
#define F(T, m) printf(#T "." #m " %zu\n", offsetof(T, m))
int main(void) {
  printf("attn_desc %zu\nattn_args %zu\nattn_caps %zu\nattn_plan_info %zu\nattn_prefill_desc %zu\n",
         sizeof(attn_desc), sizeof(attn_args), sizeof(attn_caps), sizeof(attn_plan_info), sizeof(attn_prefill_desc));
  F(attn_desc, k_page_stride); F(attn_desc, v_head_stride); F(attn_desc, sm_scale); F(attn_desc, causal);
  F(attn_args, num_pages); F(attn_args, workspace_bytes); F(attn_args, out); F(attn_args, batch);
  F(attn_caps, geometries); F(attn_plan_info, partition_max); F(attn_plan_info, split_bytes);
  F(attn_prefill_desc, q_token_stride); F(attn_prefill_desc, o_head_stride); F(attn_prefill_desc, sm_scale);
  F(attn_prefill_desc, causal);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                                 check=True).stdout.splitlines())
    assert int(got["attn_desc"]) == ctypes.sizeof(A.attn_desc)
    assert int(got["attn_args"]) == ctypes.sizeof(A.attn_args)
    assert int(got["attn_caps"]) == ctypes.sizeof(A.attn_caps)
    assert int(got["attn_plan_info"]) == ctypes.sizeof(A.attn_plan_info)
    assert int(got["attn_prefill_desc"]) == ctypes.sizeof(A.attn_prefill_desc)
    for key, val in got.items():
        if "." in key:
            struct, field = key.split(".")
            assert getattr(getattr(A, struct), field).offset == int(val), key


def test_plain_c_caller_links_and_plans(tmp_path):
    # A C99 program linked against libattn.so: capabilities, a host-only plan of the B8 x 131072
    # contract, its split policy and workspace size, and a rejected contract - no Python involved.
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "attn.h"
int main(void) {
  attn_caps caps;
  if (attn_get_capabilities(&caps) != ATTN_OK || caps.abi_version != ATTN_ABI_VERSION) return 1;
  attn_desc d;
  memset(&d, 0, sizeof d);
  d.abi_version = ATTN_ABI_VERSION; d.kv_dtype = ATTN_KV_E4M3; d.q_len = 8; d.num_q_heads = 24;
  d.num_kv_heads = 4; d.head_dim = 256; d.page_size = 1648; d.max_pages_per_seq = 80;
  d.max_seq_len = 131072; d.batch_capacity = 8;
  d.k_token_stride = d.v_token_stride = 4 * 256; d.k_head_stride = d.v_head_stride = 256;
  d.k_page_stride = d.v_page_stride = 1648LL * 4 * 256; d.causal = 1;
  attn_plan_t plan = NULL;
  size_t ws = 0;
  if (attn_plan(&d, ATTN_DEVICE_HOST_ONLY, &plan, &ws) != ATTN_OK || !plan) return 2;
  int32_t s = 0, len = 0;
  if (attn_plan_splits(plan, 131072, &s, &len) != ATTN_OK) return 3;
  printf("splits %d %d workspace %zu %zu\n", s, len, ws, attn_plan_workspace_bytes(plan, 8));
  attn_plan_destroy(plan);
  d.page_size = 1000;                            /* not a multiple of 16 */
  attn_status bad = attn_plan(&d, ATTN_DEVICE_HOST_ONLY, &plan, &ws);
  printf("bad %d %s %d\n", (int)bad, attn_status_string(bad), plan == NULL);
  return 0;
}
''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(A.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe), "-L", libdir,
                    "-lattn", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert out[:3] == ["splits", "16", "8192"]
    assert int(out[4]) == int(out[5]) == plan().workspace_bytes(8)
    assert " ".join(out[6:]) == f"bad {A.ATTN_E_INVALID} {A.status_string(A.ATTN_E_INVALID)} 1"


def test_capabilities():
    caps = A.capabilities()
    assert caps["abi_version"] == A.ATTN_ABI_VERSION
    assert caps["accumulation_bits"] == 32
    assert caps["page_alignment"] == 16
    assert caps["max_seq_len"] == 262144
    assert caps["max_batch"] >= 32
    assert {"kv_dtype": A.ATTN_KV_E4M3, "head_dim": 256, "max_q_len": 8, "max_rows": 48} in caps["geometries"]
    assert {"kv_dtype": A.ATTN_KV_FP16, "head_dim": 128, "max_q_len": 8, "max_rows": 48} in caps["geometries"]
    assert {"kv_dtype": A.ATTN_KV_E5M2, "head_dim": 256, "max_q_len": 8, "max_rows": 48} in caps["geometries"]
    assert {"kv_dtype": A.ATTN_KV_FP16, "head_dim": 256, "max_q_len": 8, "max_rows": 48} in caps["geometries"]
    assert {"kv_dtype": A.ATTN_KV_E4M3, "head_dim": 128, "max_q_len": 8, "max_rows": 48} in caps["geometries"]


def test_status_strings():
    for s in range(6):
        assert A.status_string(s)
    assert "static" in A.status_string(A.ATTN_E_STATIC_WORKSPACE)
    assert A.status_string(99) == "unknown status"


BASE = dict(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648, max_seq_len=131072,
            batch_capacity=8)


def plan(**kw):
    args = dict(BASE)
    args.update(kw)
    return A.Plan(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=1650), A.ATTN_E_INVALID),
    (dict(page_size=0), A.ATTN_E_INVALID),
    (dict(num_q_heads=25), A.ATTN_E_INVALID),
    (dict(max_seq_len=262145), A.ATTN_E_INVALID),
    (dict(max_seq_len=0), A.ATTN_E_INVALID),
    (dict(batch_capacity=0), A.ATTN_E_INVALID),
    (dict(batch_capacity=100000), A.ATTN_E_INVALID),
    (dict(max_pages_per_seq=10), A.ATTN_E_INVALID),
    (dict(k_strides=(1648 * 1024, 1024, 252)), A.ATTN_E_INVALID),      # head stride not 8-aligned
    (dict(v_strides=(0, 1024, 256)), A.ATTN_E_INVALID),
    (dict(sm_scale=float("nan")), A.ATTN_E_INVALID),
    (dict(sm_scale=-1.0), A.ATTN_E_INVALID),
    (dict(sm_scale=float("inf")), A.ATTN_E_INVALID),
    (dict(abi_version=2), A.ATTN_E_INVALID),
    (dict(kv_dtype="e3m4"), A.ATTN_E_INVALID),                         # not a KV dtype of the ABI
    (dict(kv_dtype="e5m2", head_dim=128), A.ATTN_E_UNSUPPORTED),       # E5M2 at D128 is not built
    (dict(head_dim=64), A.ATTN_E_UNSUPPORTED),                        # E4M3 at D64 is not built
    (dict(kv_dtype="fp16", head_dim=64), A.ATTN_E_UNSUPPORTED),         # FP16 at D64 is not built
    (dict(q_len=9, num_q_heads=4, num_kv_heads=4), A.ATTN_E_UNSUPPORTED),
    (dict(num_q_heads=28), A.ATTN_E_UNSUPPORTED),                       # G = 7 -> 56 rows > 48
])
def test_admission_rejects(kw, status):
    with pytest.raises(A.AttnError) as e:
        plan(**kw)
    assert e.value.status == status


@pytest.mark.parametrize("kw", [
    dict(), dict(page_size=16), dict(page_size=3296, max_seq_len=262144), dict(q_len=1, num_q_heads=4),
    dict(q_len=8, num_q_heads=4, num_kv_heads=1), dict(causal=False), dict(sm_scale=0.125),
    dict(k_strides=(1648 * 2056, 2056, 512), v_strides=(1648 * 2056, 2056, 512)),   # interleaved, 8-aligned
    dict(kv_dtype="fp16", head_dim=128, q_len=1, num_q_heads=32, num_kv_heads=8),
    dict(kv_dtype="e5m2"),
    dict(kv_dtype="fp16"),                                                 # FP16 at D256
    dict(head_dim=128),                                                    # E4M3 at D128
])
def test_admission_accepts(kw):
    p = plan(**kw)
    assert p.info["num_cus"] == 256          # host-only plans assume an MI355X
    assert p.workspace_bytes(1) * p.batch_capacity == p.workspace_bytes_capacity


def test_host_only_plan_cannot_run():
    p = plan()
    args = A.attn_args()
    assert A.lib().attn_run(p.handle, ctypes.byref(args), None) == A.ATTN_E_INVALID
    assert A.lib().attn_combine(p.handle, ctypes.byref(args), None) == A.ATTN_E_INVALID
    assert A.lib().attn_run(None, ctypes.byref(args), None) == A.ATTN_E_INVALID
    assert A.lib().attn_run(p.handle, None, None) == A.ATTN_E_INVALID


def test_null_and_bad_arguments():
    lib = A.lib()
    assert lib.attn_get_capabilities(None) == A.ATTN_E_INVALID
    h = ctypes.c_void_p()
    assert lib.attn_plan(None, -1, ctypes.byref(h), None) == A.ATTN_E_INVALID
    assert lib.attn_plan_get_info(None, None) == A.ATTN_E_INVALID
    assert lib.attn_plan_workspace_bytes(None, 1) == 0
    p = plan()
    assert lib.attn_plan_workspace_bytes(p.handle, 0) == 0
    assert lib.attn_plan_workspace_bytes(p.handle, 9) == 0
    lib.attn_plan_destroy(None)


# ---- split policy: a function of the row length and plan constants only ----

LENGTHS = [0, 1, 7, 8, 16, 255, 256, 511, 512, 513, 1024, 3297, 8191, 16384, 32768, 32769, 100000,
           131072, 200001, 262143, 262144]


def test_partitions_cover_each_row_exactly():
    p = plan(max_seq_len=262144, page_size=3296)
    info = p.info
    for L in LENGTHS:
        S, P = p.splits(L)
        if L == 0:
            assert S == 0
            continue
        assert P % info["partition_align"] == 0 and P % 32 == 0
        assert P >= info["partition_min"]
        assert (S - 1) * P < L <= S * P
        assert 1 <= S <= 64 and S <= info["grid_splits"]
        if L <= 131072:
            assert S <= info["split_cap"]
        else:
            assert P <= max(info["partition_max"], -(-L // 64))
        assert P <= 32768


def test_grid_covers_every_length():
    p = plan(max_seq_len=262144, page_size=3296)
    gs = p.info["grid_splits"]
    assert max(p.splits(L)[0] for L in range(0, 262145, 97)) <= gs
    assert max(p.splits(L)[0] for L in LENGTHS) <= gs


@pytest.mark.parametrize("hkv,cap", [(1, 64), (2, 32), (4, 16), (8, 8), (32, 8)])
def test_split_cap_follows_the_head_geometry(hkv, cap):
    p = plan(num_q_heads=hkv * 6, num_kv_heads=hkv, max_seq_len=262144, page_size=3296)
    assert p.info["split_cap"] == cap
    assert p.info["partition_max"] == 131072 // cap
    for L in LENGTHS:
        S, P = p.splits(L)
        assert S <= (cap if L <= 131072 else 64) and P <= 32768


def test_split_policy_ignores_batch_and_page_size():
    a = plan(batch_capacity=1)
    b = plan(batch_capacity=16, page_size=16)
    c = plan(batch_capacity=8, page_size=3296, max_seq_len=131072)
    for L in LENGTHS[:-2]:
        assert a.splits(L) == b.splits(L) == c.splits(L)


def test_long_rows_fill_the_chip():
    # B8 x 128K at Hkv 4: 8*4*S(131072) two-wave workgroups, one wave per SIMD of 256 CUs
    p = plan()
    S, P = p.splits(131072)
    assert 8 * 4 * S * 2 == 4 * 256
    assert P == 8192


def test_longer_rows_keep_the_128k_partition():
    # rows past 131072 tokens get more splits of the 131072-token row's partition length, so a
    # 262144-token row in a mixed batch runs no longer per workgroup than a 131072-token row
    p = plan(max_seq_len=262144, page_size=3296)
    assert p.splits(131072) == (16, 8192)
    assert p.splits(131073) == (17, 8192)
    assert p.splits(262144) == (32, 8192)
    assert p.info["grid_splits"] == 32
    # at Hkv 1 the 64-split ceiling governs: 262144 / 64 = 4096 tokens, as before
    one = plan(num_q_heads=6, num_kv_heads=1, max_seq_len=262144, page_size=3296)
    assert one.splits(262144) == (64, 4096) and one.info["grid_splits"] == 64


def test_workspace_panel_holds_the_row_tiles():
    # rows are held in tiles of 16: 48 rows at q8 G6, 16 rows at q1 G4 (D128)
    big = plan()
    small = plan(kv_dtype="fp16", head_dim=128, q_len=1, num_q_heads=32, num_kv_heads=8)
    assert big.info["rows"] == 48 and small.info["rows"] == 4
    assert big.info["split_bytes"] == -(-(48 * 256 + 96) * 4 // 256) * 256
    assert small.info["split_bytes"] == -(-(16 * 128 + 32) * 4 // 256) * 256


def test_workspace_is_request_major():
    p = plan()
    per_slot = p.workspace_bytes(1)
    assert per_slot == 4 * p.info["grid_splits"] * p.info["split_bytes"]
    assert p.info["split_bytes"] % 256 == 0
    assert p.info["split_bytes"] >= (48 * 256 + 96) * 4
    for b in range(1, 9):
        assert p.workspace_bytes(b) == b * per_slot


# ---- long prefill: admission is host-only, so it can be checked without a GPU ----

def _pf_desc(**kw):
    base = dict(abi_version=A.ATTN_ABI_VERSION, q_len=100, kv_len=300, num_q_heads=12, num_kv_heads=2, head_dim=256,
                q_token_stride=12 * 256, q_head_stride=256, k_token_stride=2 * 256, k_head_stride=256,
                v_token_stride=2 * 256, v_head_stride=256, o_token_stride=12 * 256, o_head_stride=256,
                sm_scale=0.0, causal=1)
    base.update(kw)
    return A.attn_prefill_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=128), A.ATTN_E_UNSUPPORTED),
    (dict(num_q_heads=10), A.ATTN_E_UNSUPPORTED),          # G = 5 does not divide the 12 row tiles
    (dict(num_q_heads=13), A.ATTN_E_INVALID),              # Hq % Hkv != 0
    (dict(q_len=0), A.ATTN_E_INVALID),
    (dict(kv_len=0), A.ATTN_E_INVALID),
    (dict(k_token_stride=2 * 256 + 4), A.ATTN_E_INVALID),  # not a multiple of 8 elements
    (dict(causal=2), A.ATTN_E_INVALID),
    (dict(sm_scale=-1.0), A.ATTN_E_INVALID),
    (dict(sm_scale=float("nan")), A.ATTN_E_INVALID),
    (dict(abi_version=7), A.ATTN_E_INVALID),
    (dict(k_token_stride=1 << 26), A.ATTN_E_INVALID),      # 64-key block offsets would overflow 32 bits
])
def test_prefill_admission_rejects(kw, status):
    d = _pf_desc(**kw)
    assert A.lib().attn_prefill(ctypes.byref(d), 4096, 8192, 12288, 16384, None) == status


def test_prefill_rejects_null_and_misaligned_pointers():
    d = _pf_desc()
    lib = A.lib()
    assert lib.attn_prefill(None, 4096, 8192, 12288, 16384, None) == A.ATTN_E_INVALID
    assert lib.attn_prefill(ctypes.byref(d), 0, 8192, 12288, 16384, None) == A.ATTN_E_INVALID
    assert lib.attn_prefill(ctypes.byref(d), 4096 + 8, 8192, 12288, 16384, None) == A.ATTN_E_INVALID


# ---- host-side checks of run(): caches must hold every byte the kernels may touch ----

def test_cache_extent_and_buffer_checks():
    import torch
    p = plan(page_size=32, num_q_heads=12, num_kv_heads=2, max_seq_len=4096)
    ks = (32 * 2 * 256, 2 * 256, 256)
    # last byte of the last head row of the last page, for a contiguous cache: exactly its size
    assert p.cache_extent_bytes(10, ks) == 10 * 32 * 2 * 256
    # interleaved rows (K and V of a token-head pair 520 bytes apart): D bytes past the last row start
    assert p.cache_extent_bytes(3, (32 * 2 * 520, 2 * 520, 520)) == 2 * 32 * 2 * 520 + 31 * 2 * 520 + 520 + 256
    p.device = torch.device("cpu")       # exercise the checks with host tensors
    k = torch.zeros(10, 32, 2, 256, dtype=torch.uint8)
    scale = torch.ones(1, dtype=torch.float32)
    p._validate_caches(k, k, scale, scale, 10)
    with pytest.raises(ValueError, match="holds"):
        p._validate_caches(k[:9], k, scale, scale, 10)
    with pytest.raises(ValueError, match="float32"):
        p._validate_caches(k, k, scale.double(), scale, 10)
    with pytest.raises(ValueError, match="float32"):
        p._validate_caches(k, k, scale, torch.ones(0, dtype=torch.float32), 10)
    p._validate_caches(12345, 67890, scale, scale, 10)     # raw addresses: the caller vouches


def test_run_static_refuses_host_only_plans_and_null_args():
    # Host checks only: a host-only plan or a missing argument block is refused before the
    # library looks up its static array or launches anything.
    p = A.Plan(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648, max_seq_len=131072,
               batch_capacity=8)
    args = A.attn_args()
    args.batch = 1
    assert A.lib().attn_run_static(p.handle, ctypes.byref(args), None) == A.ATTN_E_INVALID
    assert A.lib().attn_run_static(p.handle, None, None) == A.ATTN_E_INVALID
    assert A.lib().attn_run_static(None, ctypes.byref(args), None) == A.ATTN_E_INVALID


def test_static_workspace_covers_the_b8_ctx128k_contract():
    # The static array (64 MiB) holds the split panels of 8 rows of 131072 tokens at Hkv 4, D 256,
    # 48 packed rows; 16 rows of up to 262144 tokens need more and are refused on the GPU.
    p = A.Plan(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648, max_seq_len=131072,
               batch_capacity=8)
    assert p.workspace_bytes(8) <= A.ATTN_STATIC_WORKSPACE_BYTES
    big = A.Plan(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=3296, max_seq_len=262144,
                 batch_capacity=16)
    assert big.workspace_bytes(16) > A.ATTN_STATIC_WORKSPACE_BYTES
