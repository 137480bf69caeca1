"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/i8gs.h declares, and rejects invalid arguments before
touching the device (each rejection is a pure host decision)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i8gs.h")


@pytest.fixture(scope="module")
def lib():
    import int8_group_scaled_amd as i8
    return i8.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    import int8_group_scaled_amd as i8
    assert _declared_functions() == sorted(i8.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    path = os.path.join(ROOT, "int8_group_scaled_amd", "libi8gs.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_and_strings(lib):
    import int8_group_scaled_amd as i8
    assert i8.abi_version() == 1
    assert lib.i8gs_status_string(2) == b"I8GS_ERR_UNSUPPORTED_SHAPE"
    assert lib.i8gs_status_string(99) == b"I8GS_ERR_UNKNOWN"


# A 16-byte aligned host buffer stands in for device pointers: every call below is
# rejected during validation, before any pointer is dereferenced or HIP is called.
_buf = (ctypes.c_uint8 * 4096)()
_base = (ctypes.addressof(_buf) + 15) & ~15
A = ctypes.c_void_p(_base)
MIS = ctypes.c_void_p(_base + 4)
NUL = None


def _w8a8(lib, x=A, ldx=512, qa=NUL, a_s=NUL, qw=A, ws=A, y=A, ldy=256, M=8, N=256, K=512, kernel=0, split=0,
          work=A, wbytes=1 << 30):
    return lib.gemm_w8a8_g128_ex(x, ldx, qa, a_s, qw, ws, y, ldy, M, N, K, kernel, split, work, wbytes, NUL)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(K=500, ldx=504), 2, "multiple of the 128-wide"),
    (dict(K=0, ldx=0), 2, "multiple of the 128-wide"),
    (dict(N=250, ldy=256), 2, "multiple of 8"),
    (dict(M=-1), 2, ">= 0"),
    (dict(M=1 << 31), 2, "below 2^31"),
    (dict(ldx=500), 2, "ldx"),
    (dict(ldy=128), 2, "ldy"),
    (dict(qa=A, a_s=A), 1, "not both or neither"),
    (dict(x=NUL), 1, "not both or neither"),
    (dict(qw=NUL), 1, "qweight is NULL"),
    (dict(ws=NUL), 1, "w_scale is NULL"),
    (dict(y=MIS), 3, "y is not 16-byte aligned"),
    (dict(x=MIS), 3, "x is not 16-byte aligned"),
    (dict(work=NUL), 4, "workspace"),
    (dict(wbytes=16), 4, "workspace"),
    (dict(kernel=7), 1, "I8GS_KERNEL"),
    (dict(split=-2), 1, "decode_workgroups"),
    (dict(kernel=1, M=65), 2, "decode kernel"),
    (dict(kernel=1, ldy=1 << 28), 2, "R*ldy*2"),
    # 7 rows at ldy = 2^27: M*ldy*2 < 2^31, but the 32 rows the decode kernel pads to are not
    (dict(kernel=1, M=7, ldy=1 << 27), 2, "R*ldy*2"),
    (dict(kernel=1, M=40, ldy=(1 << 24) + 8), 2, "R*ldy*2"),
])
def test_w8a8_validation(lib, kwargs, status, needle):
    rc = _w8a8(lib, **kwargs)
    assert rc == status
    msg = lib.i8gs_last_error().decode()
    assert needle in msg, msg


def test_empty_inputs_are_noops(lib):
    assert _w8a8(lib, M=0) == 0
    assert _w8a8(lib, N=0, ldy=0) == 0
    assert lib.quant_act_per_token(A, 512, 0, 512, A, A, NUL) == 0
    assert lib.gemm_w4a16_g128(A, 512, A, A, A, 256, 0, 256, 512, NUL, 0, NUL) == 0


def test_quant_validation(lib):
    assert lib.quant_act_per_token(A, 512, 4, 500, A, A, NUL) == 2
    assert lib.quant_act_per_token(A, 504, 4, 512, A, A, NUL) == 2
    assert lib.quant_act_per_token(NUL, 512, 4, 512, A, A, NUL) == 1
    assert lib.quant_act_per_token(A, 512, 4, 512, MIS, A, NUL) == 3
    assert lib.quant_act_per_token(A, 512, 4, 0, A, A, NUL) == 2


def test_partials_validation(lib):
    f = lib.gemm_w8a8_g128_group_partials_ex
    assert f(A, A, NUL, 8, 256, 512, 0, 0, NUL) == 1
    assert f(A, A, A, 8, 256, 500, 0, 0, NUL) == 2
    assert f(A, A, A, 8, 256, 512, 5, 0, NUL) == 1
    assert f(A, A, A, 8, 256, 512, 0, -1, NUL) == 1
    assert f(A, A, A, 65, 256, 512, 1, 0, NUL) == 2
    assert "decode kernel" in lib.i8gs_last_error().decode()
    assert f(MIS, A, A, 8, 256, 512, 0, 0, NUL) == 3
    assert f(A, A, A, 0, 256, 512, 0, 0, NUL) == 0


def test_w4a16_activation_offsets(lib):
    """A chunk of up to 64 activation rows is addressed with 32-bit byte offsets."""
    assert lib.gemm_w4a16_g128(A, 1 << 25, A, A, A, 256, 64, 256, 512, A, 1 << 30, NUL) == 2
    assert "ldx" in lib.i8gs_last_error().decode()
    assert lib.gemm_w4a16_g128(A, 1 << 25, A, A, A, 256, 1, 256, 512, A, 1 << 30, NUL) not in (2,)


def test_w4a16_and_utility_validation(lib):
    assert lib.gemm_w4a16_g128(A, 512, A, A, A, 256, 8, 256, 384 + 64, A, 1 << 30, NUL) == 2
    assert lib.gemm_w4a16_g128(A, 512, NUL, A, A, 256, 8, 256, 512, A, 1 << 30, NUL) == 1
    assert lib.gptq_unpack(A, A, 5, 512, 256, A, NUL, NUL) == 1
    assert lib.gptq_unpack(A, A, 8, 512, 256, NUL, NUL, NUL) == 1
    assert lib.gptq_unpack(A, NUL, 8, 512, 256, NUL, A, NUL) == 1
    assert lib.gptq_unpack(A, A, 4, 200, 256, A, NUL, NUL) == 2
    assert lib.gptq_quantize_rtn(A, 3, 512, 256, A, A, NUL) == 1
    assert lib.gptq_quantize_rtn(A, 8, 512, 12, A, A, NUL) == 2
    assert lib.gemm_w8a8_g128_group_partials(A, A, NUL, 8, 256, 512, NUL) == 1


def test_workspace_sizes(lib):
    import int8_group_scaled_amd as i8
    # 64 KiB of counters, then the quantised activations (M*K + 4*M, each rounded to 256 bytes)
    assert i8.workspace_bytes(i8.OP_W8A8, 8, 256, 512, i8.KERNEL_TILED) == 65536 + 4096 + 256
    assert i8.workspace_bytes(i8.OP_W8A8, 0, 256, 512) == 0
    with pytest.raises(ValueError):
        i8.workspace_bytes(i8.OP_W8A8, 8, 256, 500)
    with pytest.raises(ValueError):
        i8.workspace_bytes(7, 8, 256, 512)
    # decode kernel, wide layer (no K split): counters and quantised activations only
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 6144, 5120, i8.KERNEL_DECODE, 3) == 65536 + 64 * 5120 + 256
    # narrow layer: 256 target workgroups on N=512 -> S=8 K parts x T=32 tiles of 16 columns:
    # one fp32 piece of 64 rows x 32 columns (the chunk width rounded up to 32) per workgroup
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 512, 5120, i8.KERNEL_DECODE, 256) == (
        65536 + 64 * 5120 + 256 + 32 * 8 * 64 * 32 * 4)


def test_prefill_split_workspace(lib):
    """Prefill (M > 64, 256 x 256 tiles, one workgroup per CU; without a GPU the CU count is
    taken as 256): the tiles of a last, partial round are split S = min(4, (K/128)/16,
    256/tail) ways (no split below 2), each split an fp32 256 x 256 piece after the counters
    and quantised activations."""
    import int8_group_scaled_amd as i8
    piece = 256 * 256 * 4
    base = lambda M, K: 65536 + M * K + 4 * M  # M*K and 4*M are multiples of 256 here
    # down: 16 x 20 = 320 tiles -> 256 whole + 64 split 4 ways
    assert i8.workspace_bytes(i8.OP_W8A8, 4096, 5120, 17408) == base(4096, 17408) + 64 * 4 * piece
    # o_proj: the same tiles, 32 groups -> 2 ways
    assert i8.workspace_bytes(i8.OP_W8A8, 4096, 5120, 4096) == base(4096, 4096) + 64 * 2 * piece
    # qkv: 16 x 24 = 384 tiles -> 128 split 2 ways
    assert i8.workspace_bytes(i8.OP_W8A8, 4096, 6144, 5120) == base(4096, 5120) + 128 * 2 * piece
    # exactly two rounds (16 x 32 tiles): nothing split
    assert i8.workspace_bytes(i8.OP_W8A8, 4096, 8192, 5120) == base(4096, 5120)
    # fewer than 32 groups cannot be split
    assert i8.workspace_bytes(i8.OP_W8A8, 4096, 5120, 3968) == base(4096, 3968)
    # two tiles split 4 ways; the tiled kernel needs no pieces
    assert i8.workspace_bytes(i8.OP_W8A8, 128, 512, 8192) == base(128, 8192) + 2 * 4 * piece
    assert i8.workspace_bytes(i8.OP_W8A8, 128, 512, 8192, i8.KERNEL_TILED) == base(128, 8192)


def test_noalloc_validation(lib):
    """The no-allocation entry point validates like gemm_w8a8_g128 and rejects, before any
    HIP call, a call whose scratch needs exceed its 16 MiB static array."""
    f = lib.gemm_w8a8_g128_noalloc
    assert lib.i8gs_noalloc_scratch_bytes() == 16 << 20
    # x given: 64 KiB + 4096*5120 quantised activations > 16 MiB
    assert f(A, 5120, NUL, NUL, A, A, A, 256, 4096, 256, 5120, NUL) == 4
    assert "16777216" in lib.i8gs_last_error().decode()
    assert f(A, 512, A, A, A, A, A, 256, 8, 256, 512, NUL) == 1   # x and qa both given
    assert f(A, 500, NUL, NUL, A, A, A, 256, 8, 256, 512, NUL) == 2
    assert f(A, 512, NUL, NUL, A, A, MIS, 256, 8, 256, 512, NUL) == 3
    assert f(A, 512, NUL, NUL, A, A, A, 256, 0, 256, 512, NUL) == 0


def test_weight_only_validation(lib):
    f = lib.gemm_weight_only
    # (bits, group): 4/128, 8/128 and 8/32 only
    assert f(A, 512, A, 4, A, 32, A, 256, 8, 256, 512, A, 1 << 30, NUL) == 1
    assert "group" in lib.i8gs_last_error().decode()
    assert f(A, 512, A, 6, A, 128, A, 256, 8, 256, 512, A, 1 << 30, NUL) == 1
    assert f(A, 512, A, 8, A, 64, A, 256, 8, 256, 512, A, 1 << 30, NUL) == 1
    assert f(A, 512, A, 8, A, 32, A, 256, 8, 250, 512, A, 1 << 30, NUL) == 2
    assert f(A, 1 << 25, A, 8, A, 32, A, 256, 64, 256, 512, A, 1 << 30, NUL) == 2
    assert f(A, 512, A, 8, A, 32, MIS, 256, 8, 256, 512, A, 1 << 30, NUL) == 3
    assert f(A, 512, A, 8, A, 32, A, 256, 0, 256, 512, NUL, 0, NUL) == 0
    g = lib.gptq_quantize_rtn_group
    assert g(A, 8, 64, 512, 256, A, A, NUL) == 1
    assert g(A, 4, 32, 500, 256, A, A, NUL) == 2
    import int8_group_scaled_amd as i8
    # the weight-only workspace covers either bit width's kernel
    assert i8.workspace_bytes(i8.OP_WEIGHT_ONLY, 64, 6144, 5120) >= i8.workspace_bytes(i8.OP_W4A16, 64, 6144, 5120)


def test_rmsnorm_quant_validation(lib):
    f = lib.rmsnorm_quant_per_token
    assert f(A, 512, A, 1e-6, 4, 500, NUL, A, A, NUL) == 2         # K % 8
    assert f(A, 512, A, 0.0, 4, 512, NUL, A, A, NUL) == 1          # eps must be positive
    assert f(A, 512, A, -1.0, 4, 512, NUL, A, A, NUL) == 1
    assert f(A, 512, NUL, 1e-6, 4, 512, NUL, A, A, NUL) == 1       # gamma NULL
    assert f(A, 512, A, 1e-6, 4, 512, MIS, A, A, NUL) == 3         # h misaligned
    assert f(A, 40000, A, 1e-6, 4, 40000, NUL, A, A, NUL) == 2     # K past the register limit
    assert "registers" in lib.i8gs_last_error().decode()
    assert f(A, 512, A, 1e-6, 0, 512, NUL, A, A, NUL) == 0


def test_kv_codec_and_attention_validation(lib):
    kvq = lib.kv_quant_int8_block128
    assert kvq(A, 100, 4, 1, A, A, NUL) == 2        # ld < 128*H
    assert kvq(A, 256, 4, 2, MIS, A, NUL) == 3      # codes misaligned
    assert kvq(NUL, 256, 4, 2, A, A, NUL) == 1      # kv NULL
    assert kvq(A, 256, 0, 2, A, A, NUL) == 0        # empty: no-op
    assert kvq(A, 256, -1, 2, A, A, NUL) == 2
    qk = lib.attn_qk_int8
    assert qk(A, A, A, A, 0.088, 4, 16, 6, 4, A, NUL, NUL) == 2      # Hq % Hkv
    assert "multiple" in lib.i8gs_last_error().decode()
    assert qk(A, A, A, A, 0.088, 4, 16, 8, 0, A, NUL, NUL) == 2      # Hkv == 0
    assert qk(A, A, A, A, float("inf"), 4, 16, 8, 4, A, NUL, NUL) == 1
    assert qk(A, A, A, A, 0.088, 4, 16, 70000, 2, A, NUL, NUL) == 2  # grid limit on heads
    assert qk(A, A, A, A, 0.088, 1048560, 1, 64, 1, A, NUL, NUL) == 2  # rows per KV head group
    assert qk(A, A, A, A, 0.088, 4, 16, 8, 4, A, MIS, NUL) == 3      # dots misaligned
    assert qk(A, NUL, A, A, 0.088, 4, 16, 8, 4, A, NUL, NUL) == 1    # qs NULL
    assert qk(NUL, NUL, NUL, NUL, 0.088, 4, 0, 8, 4, NUL, NUL, NUL) == 0  # T == 0: no-op
    pv = lib.attn_pv_int8
    W = lib.attn_pv_int8_workspace_bytes
    assert W(8, 32768, 32, 8) > 0                                    # decode: the token blocks are split
    assert W(4096, 4096, 32, 8) == 0                                 # enough row tiles: no split
    assert W(8, 0, 32, 8) == 0 and W(0, 100, 32, 8) == 0
    assert W(8, 100, 6, 4) == ctypes.c_size_t(-1).value
    need = W(8, 32768, 32, 8)
    assert pv(A, A, A, 4, 16, 6, 4, A, NUL, NUL, NUL, 0, NUL) == 2
    assert pv(A, A, A, 4, 16, 8, 4, A, NUL, MIS, NUL, 0, NUL) == 3           # ps misaligned
    assert pv(A, NUL, A, 4, 16, 8, 4, A, NUL, NUL, NUL, 0, NUL) == 1         # vq NULL
    assert pv(NUL, NUL, NUL, 0, 16, 8, 4, NUL, NUL, NUL, NUL, 0, NUL) == 0   # Mq == 0: no-op
    assert pv(A, A, A, 4, 16, 8, 4, NUL, NUL, NUL, NUL, 0, NUL) == 1         # out NULL
    assert pv(A, A, A, 8, 32768, 32, 8, A, NUL, NUL, NUL, 0, NUL) == 4       # workspace missing
    assert pv(A, A, A, 8, 32768, 32, 8, A, NUL, NUL, A, need - 1, NUL) == 4  # workspace too small
    assert pv(A, A, A, 8, 32768, 32, 8, A, NUL, NUL, MIS, need, NUL) == 3    # workspace misaligned


def test_decode_plan_on_tensor_parallel_shares(lib):
    """Decode (M = 64) on one GPU's share at tensor-parallel size 4, read off the workspace
    (without a GPU the CU count is taken as 256): where neither whole-fragment width keeps
    its groups per split at the full grid, the K splits are capped -- 64-column tiles with
    at least 8 groups per split (G/2 when K is shorter), else 128-column tiles with at least
    16 -- and each split writes one fp32 piece of 64 rows x the chunk width."""
    import int8_group_scaled_amd as i8
    base = lambda K: 65536 + 64 * K + 256  # counters, then the quantised activations
    piece = lambda tn: 64 * tn * 4
    # qkv share (N = 1536, 40 groups): 24 tiles of 64 columns x 5 splits of 8 groups
    # (the plain split would be 32 x 8 of 48 columns)
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 1536, 5120) == base(5120) + 24 * 5 * piece(64)
    # o_proj share (K = 1024, 8 groups): 80 tiles of 64 columns x 2 splits of 4 groups
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 5120, 1024) == base(1024) + 80 * 2 * piece(64)
    # gate/up share (N = 8704): no 64-column split fits; 68 tiles of 128 columns x 2 splits
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 8704, 5120) == base(5120) + 68 * 2 * piece(128)
    # down share (K = 4352, 34 groups): the whole-fragment rule already applies, 80 x 3
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 5120, 4352) == base(4352) + 80 * 3 * piece(64)
    # the four drafter layers: qkv 48 x 4 of 128 columns (10 groups per split: the rule for
    # 128-column tiles with at least 4 splits filling three quarters of the grid), o_proj
    # 80 x 3, down 40 x 6 of 128 columns, gate_up unsplit
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 6144, 5120) == base(5120) + 48 * 4 * piece(128)
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 5120, 4096) == base(4096) + 80 * 3 * piece(64)
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 5120, 17408) == base(17408) + 40 * 6 * piece(128)
    assert i8.workspace_bytes(i8.OP_W8A8, 64, 34816, 5120) == base(5120)


def test_weight_only_plan_on_the_decode_layers(lib):
    """The LDS-staged weight-only kernel's grid, read off the workspace (256 CUs without a
    GPU): 128-column tiles x row chunks x K splits, one fp32 piece of 8 waves x MT*4 x 64
    lanes per workgroup.  Narrow layers (tiles x chunks at most half the CUs) take one
    workgroup per CU, floor(256 / (tiles * chunks)) splits; wider ones 1.5 per CU, or 3 per
    CU with more tiles than CUs.  The workspace covers 4- and 8-bit codes alike."""
    import int8_group_scaled_amd as i8
    part = lambda units, S, MT: units * S * 8 * MT * 4 * 64 * 4
    for op in (i8.OP_W4A16, i8.OP_WEIGHT_ONLY):
        # M = 8 (one 16-row tile): qkv 48 tiles -> 5 splits; o_proj and down 40 tiles -> 6
        assert i8.workspace_bytes(op, 8, 6144, 5120) == 65536 + part(48, 5, 1)
        assert i8.workspace_bytes(op, 8, 5120, 4096) == 65536 + part(40, 6, 1)
        assert i8.workspace_bytes(op, 8, 5120, 17408) == 65536 + part(40, 6, 1)
        # gate_up: 272 tiles, more than the CUs -> 3 per CU: ceil(768 / 272) = 3 splits
        assert i8.workspace_bytes(op, 8, 34816, 5120) == 65536 + part(272, 3, 1)
        # M = 64: qkv and down keep 64-row tiles (5 and 6 splits); o_proj, whose 6 splits
        # would leave 5 groups each, takes two 32-row chunks: 80 units -> 3 splits
        assert i8.workspace_bytes(op, 64, 6144, 5120) == 65536 + part(48, 5, 4)
        assert i8.workspace_bytes(op, 64, 5120, 17408) == 65536 + part(40, 6, 4)
        assert i8.workspace_bytes(op, 64, 5120, 4096) == 65536 + part(80, 3, 2)
