"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before touching the device."""

import ctypes
import os
import re

import pytest
import torch

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxfp4moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from mxfp4_moe_expert_route_amd import _lib
    assert os.path.exists(_lib.LIB_PATH), "library not built: run __graft_entry__.build()"
    return _lib.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mxfp4_pack", "mxfp4_unpack", "moe_route_topk", "moe_router_topk",
              "dflash_verify_accept", "dflash_verify_workspace_bytes", "moe_permute",
              "moe_permute_workspace_bytes", "moe_route_permute", "moe_mxfp4_gate_up_swiglu", "moe_mxfp4_down",
              "moe_combine", "moe_mxfp4_layer", "moe_mxfp4_layer_noalloc", "mxm_stream_xor",
              "moe_mxfp4_decode_layer", "moe_mxfp4_decode_layer_workspace_bytes",
              "mxm_status_string", "mxm_version"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    from mxfp4_moe_expert_route_amd import _lib
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings(lib):
    for s in range(-8, 1):
        assert lib.mxm_status_string(s)
    assert lib.mxm_version() >= 100


P = 256        # an aligned fake device address: never dereferenced on error paths


def test_pack_unpack_argument_checks(lib):
    assert lib.mxfp4_pack(P, 7, 4, 64, P, P, None) == -3            # dtype
    assert lib.mxfp4_pack(P, 0, 4, 48, P, P, None) == -2            # K % 32
    assert lib.mxfp4_pack(P, 0, -1, 64, P, P, None) == -2
    assert lib.mxfp4_pack(None, 0, 4, 64, P, P, None) == -1         # null
    assert lib.mxfp4_pack(P + 4, 0, 4, 64, P, P, None) == -4        # misaligned x
    assert lib.mxfp4_pack(None, 0, 0, 64, None, None, None) == 0    # empty: no-op
    assert lib.mxfp4_unpack(P, P, 4, 64, P, 9, None) == -3
    assert lib.mxfp4_unpack(P, P, 4, 33, P, 0, None) == -2
    assert lib.mxfp4_unpack(P, None, 4, 64, P, 0, None) == -1
    assert lib.mxfp4_unpack(P + 8, P, 4, 64, P, 0, None) == -4


def test_route_permute_argument_checks(lib):
    assert lib.moe_route_topk(P, 4, 8, 9, P, P, None) == -2          # k > E
    assert lib.moe_route_topk(P, 4, 1025, 8, P, P, None) == -2       # E > 1024
    assert lib.moe_route_topk(P, 4, 64, 33, P, P, None) == -2        # k > 32
    assert lib.moe_route_topk(P, 4, 8, 0, P, P, None) == -2
    assert lib.moe_route_topk(None, 4, 8, 2, P, P, None) == -1
    assert lib.moe_route_topk(P + 2, 4, 8, 2, P, P, None) == -4
    assert lib.moe_route_permute(P, 4, 8, 9, P, P, P, P, P, P, None, 0, None) == -2   # k > E
    assert lib.moe_route_permute(P, 4, 1025, 8, P, P, P, P, P, P, None, 0, None) == -2
    assert lib.moe_route_permute(P, 4, 8, 2, P, P, None, P, P, P, None, 0, None) == -1
    assert lib.moe_route_permute(P, 4, 8, 2, P, P, P, P + 2, P, P, None, 0, None) == -4
    assert lib.moe_route_permute(P, 0, 8, 2, None, None, None, None, None, None, None, 0,
                                 None) == 0
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == 0
    assert lib.moe_permute_workspace_bytes(64, 384, 8) == 0
    # above 8192 pairs: one E-int histogram per range of 1024 pairs
    assert lib.moe_permute_workspace_bytes(1024, 384, 8) == 0
    assert lib.moe_permute_workspace_bytes(1025, 384, 8) == 9 * 384 * 4
    assert lib.moe_permute_workspace_bytes(8192, 384, 8) == 64 * 384 * 4
    assert lib.moe_permute_workspace_bytes(8192, 2000, 8) == 0          # E > 1024: invalid
    # a needed workspace may not be NULL
    assert lib.moe_permute(P, 8192, 384, 8, P, P, P, P, None, 64 * 384 * 4, None) == -1
    assert lib.moe_permute(P, 4, 8, 2, P, P, P, None, None, 0, None) == -1
    assert lib.moe_permute(P, 4, 8, 9, P, P, P, P, None, 0, None) == -2


def test_router_argument_checks(lib):
    # x, w_router, bias, T, H, E, k, logits, ids, w, stream
    assert lib.moe_router_topk(P, P, None, 4, 64, 8, 9, P, P, P, None) == -2     # k > E
    assert lib.moe_router_topk(P, P, None, 4, 66, 8, 2, P, P, P, None) == -2     # H % 4
    assert lib.moe_router_topk(P, P, None, 4, 0, 8, 2, P, P, P, None) == -2      # H = 0
    assert lib.moe_router_topk(P, P, None, 4, 64, 1025, 8, P, P, P, None) == -2  # E > 1024
    assert lib.moe_router_topk(None, P, None, 4, 64, 8, 2, P, P, P, None) == -1  # null x
    assert lib.moe_router_topk(P, P, None, 4, 64, 8, 2, None, P, P, None) == -1  # null logits
    assert lib.moe_router_topk(P + 4, P, None, 4, 64, 8, 2, P, P, P, None) == -4  # x 8-byte
    assert lib.moe_router_topk(P, P + 8, None, 4, 64, 8, 2, P, P, P, None) == -4  # w 16-byte
    assert lib.moe_router_topk(P, P, P + 2, 4, 64, 8, 2, P, P, P, None) == -4     # bias
    assert lib.moe_router_topk(None, None, None, 0, 64, 8, 2, None, None, None, None) == 0


def test_verify_argument_checks(lib):
    ws = lib.dflash_verify_workspace_bytes(4, 8, 64)
    assert ws > 0 and lib.dflash_verify_workspace_bytes(4, 33, 64) == 0
    # target, draft, tokens, uniforms, B, L, V, accept_len, next_token, ws, bytes, stream
    assert lib.dflash_verify_accept(P, P, P, P, 4, 8, 50, P, P, P, ws, None) == -2      # V % 4
    assert lib.dflash_verify_accept(P, P, P, P, 4, 0, 64, P, P, P, ws, None) == -2      # L < 1
    assert lib.dflash_verify_accept(P, P, P, P, 4, 33, 64, P, P, P, ws, None) == -2     # L > 32
    assert lib.dflash_verify_accept(P, P, P, P, 4, 8, 64, P, P, P, ws - 1, None) == -7  # workspace
    assert lib.dflash_verify_accept(None, P, P, P, 4, 8, 64, P, P, P, ws, None) == -1
    assert lib.dflash_verify_accept(P + 4, P, P, P, 4, 8, 64, P, P, P, ws, None) == -4  # 16-byte
    assert lib.dflash_verify_accept(None, None, None, None, 0, 8, 64, None, None, None, 0, None) == 0


def test_ffn_combine_argument_checks(lib):
    gu = lib.moe_mxfp4_gate_up_swiglu
    assert gu(P, P, P, 8, 6160, 2048, 384, 8, P, P, P, None) == -2   # H % 32
    assert gu(P, P, P, 8, 6144, 2040, 384, 8, P, P, P, None) == -2   # I % 32
    assert gu(P, P, P, 8, 6144, 2048, 384, 400, P, P, P, None) == -2
    assert gu(P, None, P, 8, 6144, 2048, 384, 8, P, P, P, None) == -1
    assert gu(P + 8, P, P, 8, 6144, 2048, 384, 8, P, P, P, None) == -4
    assert gu(None, None, None, 0, 6144, 2048, 384, 8, None, None, None, None) == 0
    dn = lib.moe_mxfp4_down
    assert dn(P, P, 8, 6144, 2048, 384, 8, P, P, None, None) == -1
    assert dn(P, P, 8, 6144, 16, 384, 8, P, P, P, None) == -2
    assert dn(P, P, 8, 6144, 2048, 384, 8, P + 4, P, P, None) == -4
    cb = lib.moe_combine
    assert cb(P, P, P, 8, 6144, 0, P, None) == -2
    assert cb(P, P, None, 8, 6144, 8, P, None) == -1
    assert cb(P, P, P, 8, 6144, 8, P + 4, None) == -4
    assert cb(None, None, None, 0, 6144, 8, None, None) == 0


def test_python_wrappers_reject_host_tensors():
    import mxfp4_moe_expert_route_amd as mm
    with pytest.raises(ValueError):
        mm.mxfp4_pack(torch.zeros(4, 64))
    with pytest.raises(TypeError):
        mm.moe_route_topk(torch.zeros(4, 8, dtype=torch.float64), 2)


def test_noalloc_layer_argument_checks(lib):
    f = lib.moe_mxfp4_layer_noalloc
    ptrs = [P] * 13
    # 131072 tokens x top-8 over 1024 experts: 1024 ranges x 4 KB of grouping
    # workspace, beyond the fixed 1 MiB scratch
    assert f(P, P, 131072, 6144, 2048, 1024, 8, *ptrs, None) == -8
    # the largest page-shaped batch that fits: 682 ranges x 384 x 4 B <= 1 MiB;
    # one pair more needs 683 ranges
    assert lib.moe_permute_workspace_bytes(87296, 384, 8) <= 1 << 20
    assert f(P, P, 87297, 6144, 2048, 384, 8, *ptrs, None) == -8
    assert f(P, P, 0, 6144, 2048, 384, 8, *ptrs, None) == 0                 # empty: no-op
    assert f(P, P, 8, 6144, 2048, 384, 33, *ptrs, None) == -2       # k > 32
    assert f(None, P, 8, 6144, 2048, 384, 8, *ptrs, None) == -1             # null x
    assert f(P + 4, P, 8, 6144, 2048, 384, 8, *ptrs, None) == -4            # misaligned x
    # nulls are caught before the scratch is looked up, also above 8192 pairs
    assert f(None, P, 2048, 256, 128, 384, 8, *ptrs, None) == -1


def test_decode_layer_argument_checks(lib):
    nbytes = lib.moe_mxfp4_decode_layer_workspace_bytes
    f = lib.moe_mxfp4_decode_layer
    ws = nbytes(8, 6144, 2048, 384, 8)
    assert ws >= 2048
    assert nbytes(17, 6144, 2048, 384, 8) == 0          # more than 16 tokens
    assert nbytes(8, 6144, 1024, 384, 8) == 0           # I not a multiple of 2048
    assert nbytes(8, 16384, 2048, 384, 8) == 0          # H above 8192
    assert nbytes(16, 2048, 2048, 1024, 32) == ws       # T k = 512, the most it takes
    ptrs = [P] * 13
    assert f(P, P, 0, 6144, 2048, 384, 8, *ptrs, P, ws, None) == 0         # empty: no-op
    assert f(P, P, 17, 6144, 2048, 384, 8, *ptrs, P, ws, None) == -6       # not taken
    assert f(P, P, 8, 6144, 2048, 384, 8, *ptrs, P, ws - 1, None) == -7    # workspace
    assert f(P, P, 8, 6144, 2048, 384, 8, *ptrs, None, ws, None) == -1     # null workspace
    assert f(P, P, 8, 6144, 2048, 384, 8, *ptrs, P + 8, ws, None) == -4    # misaligned
    assert f(None, P, 8, 6144, 2048, 384, 8, *ptrs, P, ws, None) == -1     # null x
    assert f(P, P, 8, 6144, 2048, 384, 40, *ptrs, P, ws, None) == -2       # k > 32
