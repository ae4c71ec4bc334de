"""The C-ABI library loads, exports every entry point the header declares, and rejects
bad arguments before touching a device (so this runs without a GPU)."""
import ctypes
import os
import re

import pytest

import mxfp4_expert_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe_layer.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(moe.EXPORTS) == names


def test_expert_bytes_and_status_strings():
    assert moe.expert_bytes(3584, 3072) == 17_547_264
    assert moe.expert_bytes(128, 128) == 26_112
    assert moe.expert_bytes(100, 128) == 0
    for s, name in moe.STATUS.items():
        assert moe.lib().moe_status_string(s).decode() == name


FAKE = 0x7F0000000000  # a 16-byte aligned address; never dereferenced on these paths


def k3(T=1, **kw):
    c = dict(num_tokens=T, d_model=7168, d_latent=3584, d_ffn=3072, num_experts=896)
    c.update(kw)
    return moe.MoEConfig(c["num_tokens"], c["d_model"], c["d_latent"], c["d_ffn"], c["num_experts"],
                         kw.get("act", 0), kw.get("renormalize", 1), kw.get("bias_row_stride", 0),
                         kw.get("expert_layout", 0), kw.get("act_format", 0), kw.get("num_shared", 0),
                         kw.get("d_ffn_shared", 0))


def ws_status(cfg, k):
    n = ctypes.c_size_t(0)
    return moe.lib().moe_workspace_size(ctypes.byref(cfg), k, ctypes.byref(n)), n.value


def test_workspace_size_valid_and_invalid():
    st, n = ws_status(k3(T=4096), 16)
    assert st == 0 and n > 4096 * 16 * 3072 * 2
    assert ws_status(k3(), 0)[0] == -1            # k < 1
    assert ws_status(k3(), 65)[0] == -1           # k > 64
    assert ws_status(k3(num_experts=8), 9)[0] == -1  # k > E
    assert ws_status(k3(d_latent=100), 16)[0] == -1  # not a multiple of 32
    assert ws_status(k3(d_latent=3616), 16)[0] == -2  # multiple of 32, not of 128: unsupported here
    assert ws_status(k3(act=1), 16)[0] == -2      # SiTU not defined on the pages
    assert ws_status(k3(act=7), 16)[0] == -1
    assert ws_status(k3(renormalize=2), 16)[0] == -1
    assert ws_status(k3(bias_row_stride=5), 16)[0] == -1
    assert ws_status(k3(num_experts=2048), 16)[0] == -2
    assert ws_status(k3(T=-1), 16)[0] == -1
    assert ws_status(k3(expert_layout=1), 16)[0] == 0
    assert ws_status(k3(expert_layout=2), 16)[0] == -1
    assert ws_status(k3(act_format=1), 16)[0] == 0   # MXFP8 activations
    assert ws_status(k3(act_format=2), 16)[0] == -1
    assert ws_status(k3(num_shared=2, d_ffn_shared=3072), 16)[0] == 0
    assert ws_status(k3(num_shared=2, d_ffn_shared=3072), 16)[1] > ws_status(k3(), 16)[1]
    assert ws_status(k3(num_shared=2, d_ffn_shared=0), 16)[0] == -1
    assert ws_status(k3(num_shared=9, d_ffn_shared=3072), 16)[0] == -1
    assert ws_status(k3(num_shared=1, d_ffn_shared=3104), 16)[0] == -2  # not a multiple of 128
    assert moe.lib().moe_workspace_size(None, 16, ctypes.byref(ctypes.c_size_t())) == -1


def fwd(cfg, k=16, x=FAKE, out=FAKE + (1 << 30), ws=FAKE + (2 << 30), ws_bytes=1 << 40, **ptrs):
    p = dict(router_w=FAKE + (3 << 30), latent_down=FAKE + (4 << 30), latent_up=FAKE + (5 << 30),
             blob=FAKE + (6 << 30), bias=None)
    p.update(ptrs)
    return moe.lib().moe_layer_forward(x, p["router_w"], p["latent_down"], p["latent_up"], p["blob"], k,
                                       ctypes.byref(cfg), p["bias"], out, None, ws, ws_bytes, None)


def test_forward_argument_errors_return_before_any_launch():
    assert fwd(k3(T=0)) == 0                                  # T = 0 is a no-op
    assert fwd(k3(), x=None) == -1
    assert fwd(k3(), out=None) == -1
    assert fwd(k3(), blob=None) == -1
    assert fwd(k3(), x=FAKE + 8) == -1                         # misaligned
    assert fwd(k3(), out=FAKE) == -1                           # out aliases x
    assert fwd(k3(), k=0) == -1
    assert fwd(k3(act=1)) == -2
    assert fwd(k3(), ws=None) == -3
    assert fwd(k3(), ws_bytes=1024) == -3
    assert fwd(k3(), ws=FAKE + (2 << 30) + 8) == -1            # misaligned workspace
    assert fwd(k3(), bias=FAKE + 2) == -1                      # misaligned bias
    r = moe.RoutingOut(saliency=FAKE + 4)                      # misaligned fp64 saliency
    assert moe.lib().moe_layer_forward(FAKE, FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30), FAKE + (6 << 30),
                                       16, ctypes.byref(k3()), None, FAKE + (1 << 30), ctypes.byref(r),
                                       FAKE + (2 << 30), 1 << 40, None) == -1


def test_stage_argument_errors():
    L = moe.lib()
    assert L.moe_dequant_mxfp4(None, FAKE, 4, 64, FAKE, None) == -1
    assert L.moe_dequant_mxfp4(FAKE, FAKE, 4, 48, FAKE, None) == -1
    assert L.moe_dequant_mxfp4(FAKE, FAKE, 0, 64, FAKE, None) == 0  # empty launch
    assert L.moe_topk(FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == -1
    assert L.moe_topk(FAKE, 0, 8, 2, 1, FAKE, FAKE, None) == 0
    assert L.moe_topk(FAKE, 4, 2048, 2, 1, FAKE, FAKE, None) == -2
    assert L.moe_permute(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == -3
    assert L.moe_permute(FAKE, 0, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == 0
    n = ctypes.c_size_t(7)
    assert L.moe_permute_workspace_size(0, 2, 8, ctypes.byref(n)) == 0 and n.value == 0
    for T, k, E in ((4, 2, 8), (4096, 16, 896), (70001, 2, 8)):
        assert L.moe_permute_workspace_size(T, k, E, ctypes.byref(n)) == 0
        assert n.value > 0 and n.value % 256 == 0
        # one byte short of the size is refused before any device work
        assert L.moe_permute(FAKE, T, k, E, FAKE, FAKE, FAKE, FAKE, n.value - 1, None) == -3
    assert L.moe_permute_workspace_size(4, 9, 8, ctypes.byref(n)) == -1   # k > E
    assert L.moe_permute_workspace_size(-1, 2, 8, ctypes.byref(n)) == -1
    assert L.moe_permute_workspace_size(4, 2, 8, None) == -1
    assert L.moe_permute_workspace_size(4, 2, 4096, ctypes.byref(n)) == -2  # E past the supported maximum
    assert L.moe_combine(FAKE, FAKE, 4, 2, 100, FAKE, None) == -1
    assert L.moe_linear_bf16(FAKE, FAKE, 4, 100, 8, FAKE, None) == -1
    assert L.moe_linear_bf16(FAKE, FAKE, 0, 64, 8, FAKE, None) == 0
    r = moe.RoutingOut(None, None, None, None, None, None)
    assert L.moe_route(FAKE, FAKE, None, ctypes.byref(k3()), 16, 0, ctypes.byref(r), FAKE, 1 << 40, None) == -1
    r = moe.RoutingOut(FAKE, FAKE, FAKE, None, None, None)
    assert L.moe_route(FAKE, FAKE, None, ctypes.byref(k3()), 16, 8, ctypes.byref(r), FAKE, 1 << 40, None) == -1
    assert L.moe_expert_ffn(FAKE, FAKE, 16, ctypes.byref(k3()), None, FAKE, None, FAKE, 1 << 40, None) == -1


def test_packed_layout_sizes_and_pack_errors():
    # same bytes as the record when L and F are multiples of 512; one padded scale tile
    # per 16-row group of a matrix whose K/128 is not a multiple of 4
    assert moe.packed_expert_bytes(3584, 3072) == moe.expert_bytes(3584, 3072)
    # L = 384: gate/up groups hold 12 scale bytes per row (3 steps) in a 16-byte slot;
    # F = 256: down groups 8 in 16
    assert moe.packed_expert_bytes(384, 256) == moe.expert_bytes(384, 256) + 2 * (256 // 16) * 64 + (384 // 16) * 128
    assert moe.packed_expert_bytes(100, 128) == 0 and moe.packed_expert_bytes(160, 128) == 0
    pack = moe.lib().moe_pack_experts
    assert pack(FAKE, 0, 3584, 3072, FAKE + (1 << 40), None) == 0        # nothing to do
    assert pack(FAKE, 4, 3584, 3000, FAKE + (1 << 40), None) == -1       # F not a multiple of 128
    assert pack(FAKE, -1, 3584, 3072, FAKE + (1 << 40), None) == -1
    assert pack(None, 4, 3584, 3072, FAKE + (1 << 40), None) == -1
    assert pack(FAKE + 8, 4, 3584, 3072, FAKE + (1 << 40), None) == -1   # misaligned
    assert pack(FAKE, 4, 3584, 3072, FAKE + 4096, None) == -1            # overlapping buffers


@pytest.mark.parametrize("cname,pyname", [("moe_config", "MoEConfig"), ("moe_routing_out", "RoutingOut")])
def test_struct_layout_matches_header(tmp_path, cname, pyname):
    """The ctypes mirrors of the ABI's structs have the header's size and field offsets."""
    import subprocess
    cls = getattr(moe, pyname)
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "moe_layer.h"\nint main(void) {\n'
                   f'  printf("%zu\\n", sizeof({cname}));\n' +
                   "".join(f'  printf("%zu\\n", offsetof({cname}, {f}));\n' for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(cls)
    assert got[1:] == [getattr(cls, f).offset for f in fields]


def test_reap_keep_bias_errors_before_any_launch():
    L = moe.lib()
    assert L.moe_reap_keep_bias(None, 896, 242, FAKE, None) == -1
    assert L.moe_reap_keep_bias(FAKE, 896, 242, None, None) == -1
    assert L.moe_reap_keep_bias(FAKE, 896, 897, FAKE, None) == -1       # more kept than experts
    assert L.moe_reap_keep_bias(FAKE, 896, -1, FAKE, None) == -1
    assert L.moe_reap_keep_bias(FAKE, 0, 0, FAKE, None) == -1
    assert L.moe_reap_keep_bias(FAKE + 4, 896, 242, FAKE, None) == -1   # fp64 saliency misaligned
    assert L.moe_reap_keep_bias(FAKE, 896, 242, FAKE + 2, None) == -1   # fp32 bias misaligned
    assert L.moe_reap_keep_bias(FAKE, 2048, 242, FAKE, None) == -2      # more experts than one block ranks


def test_streamed_forward_slots_and_errors_before_any_launch():
    L = moe.lib()
    cfg = k3(T=1)
    n = ctypes.c_size_t(0)
    assert L.moe_expert_slots_bytes(ctypes.byref(cfg), 16, ctypes.byref(n)) == 0
    assert n.value == 16 * 17_547_264                      # min(E, T*k) records
    cfg64 = k3(T=64)
    assert L.moe_expert_slots_bytes(ctypes.byref(cfg64), 16, ctypes.byref(n)) == 0
    assert n.value == 896 * 17_547_264
    assert L.moe_expert_slots_bytes(ctypes.byref(cfg), 0, ctypes.byref(n)) == -1

    def sfwd(cfg, slots=FAKE + (4 << 30), slots_bytes=1 << 40, blob=FAKE + (8 << 30), k=16):
        return L.moe_layer_forward_streamed(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), blob, k,
                                            ctypes.byref(cfg), None, slots, slots_bytes, FAKE + (5 << 30), None,
                                            FAKE + (6 << 30), 1 << 40, None)
    assert sfwd(k3(T=1), slots=None) == -1
    assert sfwd(k3(T=0)) == 0
    assert sfwd(k3(T=1), slots_bytes=16 * 17_547_264 - 1) == -1   # slot buffer too small
    assert sfwd(k3(T=1), slots=FAKE + (4 << 30) + 8) == -1        # misaligned slots
    assert sfwd(k3(T=1), blob=None) == -1
    assert sfwd(k3(T=1), k=0) == -1
    shared = k3(T=1)
    shared.num_shared, shared.d_ffn_shared = 2, 3072
    assert sfwd(shared) == -2


def test_expert_ffn_binding_rejects_wrong_output_buffers():
    # the shapes of caller-given outputs are checked before anything reaches the library
    import torch
    h = torch.zeros((3, 128), dtype=torch.int16)
    idx = torch.zeros((3, 2), dtype=torch.int32)
    kw = dict(d_model=256, d_ffn=128, num_experts=8)
    with pytest.raises(ValueError):
        moe.expert_ffn(h, h, idx, y=torch.zeros((5, 128), dtype=torch.float32), **kw)
    with pytest.raises(ValueError):
        moe.expert_ffn(h, h, idx, y=torch.zeros((6, 128), dtype=torch.float64), **kw)
    with pytest.raises(ValueError):
        moe.expert_ffn(h, h, idx, y=torch.zeros((6, 128), dtype=torch.float32),
                       a=torch.zeros((6, 64), dtype=torch.int16), **kw)


def test_noalloc_refuses_batches_past_its_scratch_before_any_launch():
    """moe_layer_forward_noalloc: a batch whose workspace exceeds the library's scratch, or
    one with shared experts, is refused before the device is touched."""
    lib = moe.lib()
    big = k3(T=4096)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(big), 16, ctypes.byref(n)) == 0 and n.value > moe.NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 5
    assert lib.moe_layer_forward_noalloc(*args, 16, ctypes.byref(big), None, FAKE, None, None) == -3
    shared = k3(T=1, num_shared=2, d_ffn_shared=3072)
    assert lib.moe_layer_forward_noalloc(*args, 16, ctypes.byref(shared), None, FAKE, None, None) == -1
    assert lib.moe_layer_forward_noalloc(*args, 0, ctypes.byref(k3(T=1)), None, FAKE, None, None) == -1
