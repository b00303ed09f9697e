"""The C ABI on the host: exports, struct agreement and every argument check.

No compute call happens here: each call either queries sizes or fails its
host-side checks before anything is queued.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from gated_delta_rule_65_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def chunk_args(**kw):
    a = B.ChunkArgs()
    a.struct_size = ctypes.sizeof(B.ChunkArgs)
    a.dtype, a.num_seqs, a.total_tokens, a.hqk, a.hv = 1, 2, 256, 2, 4
    a.scale, a.use_qk_l2norm = 128 ** -0.5, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def ws_size(lib, a):
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_struct_size_agrees_and_workspace_is_sized(lib):
    st, n = ws_size(lib, chunk_args())
    assert st == B.KDA_OK and n > 0
    bad = chunk_args()
    bad.struct_size -= 8
    assert ws_size(lib, bad)[0] == B.KDA_ERR_ARG


def test_workspace_layout_is_ordered_and_covers_intermediates(lib):
    a = chunk_args(path=B.PATH_FUSED)
    lay = B.WsLayout()
    assert lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay)) == B.KDA_OK
    assert lay.max_chunks == 256 // 64 + 2
    offs = [lay.chunk_offsets, lay.zero, lay.table, lay.qg, lay.kg_t, lay.decay, lay.w, lay.u,
            lay.aqk, lay.scan]
    assert offs == sorted(offs)
    assert lay.zero - lay.chunk_offsets >= 4 * 3 and lay.table - lay.zero >= 1024
    assert lay.qg - lay.table >= 16 * lay.max_chunks
    assert lay.kg_t - lay.qg >= 256 * 4 * 128 * 2
    assert lay.total >= lay.aqk + 256 * 4 * 64 * 2
    assert all(o % 256 == 0 for o in offs)
    # groups add the scan planes: 3 planes of 128x128 fp32 per (group, seq, head)
    g = chunk_args(groups=4, path=B.PATH_FUSED)
    lay4 = B.WsLayout()
    assert lib.kda_chunk_ws_layout(ctypes.byref(g), ctypes.byref(lay4)) == B.KDA_OK
    assert lay4.total - lay4.scan >= 4 * 2 * 4 * 3 * 128 * 128 * 4


def test_onchip_workspace_holds_only_the_table_and_scan_planes(lib):
    """The on-chip path keeps no intermediate regions: only the chunk table
    and (under the group scan) the scan planes."""
    for path in (B.PATH_ONCHIP,):
        a = chunk_args(path=path, groups=1)
        lay = B.WsLayout()
        assert lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay)) == B.KDA_OK
        assert lay.qg == lay.kg_t == lay.decay == lay.w == lay.u == lay.aqk == lay.scan
        assert lay.total == lay.scan
        assert lay.scan - lay.table >= 16 * lay.max_chunks
        g = chunk_args(path=path, groups=4)
        assert lib.kda_chunk_ws_layout(ctypes.byref(g), ctypes.byref(lay)) == B.KDA_OK
        assert lay.total - lay.scan == 4 * 2 * 4 * 3 * 128 * 128 * 4
    # the on-chip path is bf16 only; AUTO keeps the staged layout
    assert ws_size(lib, chunk_args(dtype=0, path=B.PATH_ONCHIP))[0] == B.KDA_ERR_UNSUPPORTED
    for dtype in (0, 1):
        a = chunk_args(dtype=dtype)
        assert lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay)) == B.KDA_OK
        assert lay.kg_t > lay.qg


@pytest.mark.parametrize("field,value,status", [
    ("hv", 3, B.KDA_ERR_SHAPE),            # GVA divisibility
    ("hqk", 0, B.KDA_ERR_SHAPE),
    ("dtype", 9, B.KDA_ERR_DTYPE),
    ("num_seqs", -1, B.KDA_ERR_SHAPE),
    ("total_tokens", 255, B.KDA_ERR_SHAPE),  # dense: not a multiple of num_seqs
    ("scale", float("inf"), B.KDA_ERR_SHAPE),
    ("path", 7, B.KDA_ERR_UNSUPPORTED),
    ("groups", -2, B.KDA_ERR_SHAPE),
    ("groups", 65, B.KDA_ERR_UNSUPPORTED),
    ("walk_waves", 3, B.KDA_ERR_ARG),
])
def test_chunk_checks(lib, field, value, status):
    a = chunk_args(**{field: value})
    assert ws_size(lib, a)[0] == status
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == status
    assert lib.kda_last_error().decode() != ""


def test_chunk_counts_beyond_32_bits_are_rejected(lib):
    # tokens, and (chunks + sequences) x value heads, are counted in 32 bits
    for a in (chunk_args(total_tokens=2 ** 31), chunk_args(total_tokens=2 ** 30, hv=256)):
        assert ws_size(lib, a)[0] == B.KDA_ERR_UNSUPPORTED
        assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_UNSUPPORTED
    assert ws_size(lib, chunk_args(total_tokens=2 ** 30, hv=64))[0] == B.KDA_OK


def test_chunk_state_modes_are_exclusive(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the checks fail first
    a = chunk_args(state_cache=fake, initial_state=fake, num_slots=4)
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_SHAPE
    a = chunk_args(state_cache=fake, num_slots=4)          # no indices
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_SHAPE
    a = chunk_args(state_indices=fake)                     # indices without a cache
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_SHAPE
    a = chunk_args(state_cache=fake, state_indices=fake, has_initial_state=fake,
                   num_slots=0)
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_SHAPE


def test_chunk_missing_pointers_and_workspace(lib):
    a = chunk_args()                                       # q..out NULL
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_ARG
    fake = ctypes.c_void_p(0x1000)
    a = chunk_args(q=fake, k=fake, v=fake, g=fake, beta=fake, out=fake)
    _, need = ws_size(lib, a)
    a.workspace, a.workspace_bytes = fake, need - 1
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = None, need
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == B.KDA_ERR_WORKSPACE


def decode_args(**kw):
    a = B.DecodeArgs()
    a.struct_size = ctypes.sizeof(B.DecodeArgs)
    a.dtype, a.n, a.hqk, a.hv, a.scale, a.use_qk_l2norm, a.num_slots = 1, 4, 2, 4, 0.1, 1, 8
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("hv", 3, B.KDA_ERR_SHAPE),
    ("dtype", 5, B.KDA_ERR_DTYPE),
    ("n", -1, B.KDA_ERR_SHAPE),
    ("num_slots", 0, B.KDA_ERR_SHAPE),
    ("num_slots", 3, B.KDA_ERR_SHAPE),      # identity map needs n slots
    ("struct_size", 8, B.KDA_ERR_ARG),
])
def test_decode_checks(lib, field, value, status):
    a = decode_args(**{field: value})
    assert lib.kda_decode(ctypes.byref(a)) == status


def test_decode_null_pointers_and_empty_batch(lib):
    assert lib.kda_decode(ctypes.byref(decode_args())) == B.KDA_ERR_ARG
    assert lib.kda_decode(ctypes.byref(decode_args(n=0))) == B.KDA_OK   # nothing queued
    assert lib.kda_decode(None) == B.KDA_ERR_ARG


def test_status_strings(lib):
    for s in range(7):
        assert lib.kda_status_str(s).decode()
    assert b"gfx950" in lib.kda_version()


def cpu(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_binding_shape_checks_raise_like_chunk_kda():
    q = cpu((1, 64, 2, 128))
    v = cpu((1, 64, 4, 128))
    beta = cpu((1, 64, 4))
    with pytest.raises(ValueError, match="D=128"):
        B.chunk_kda(cpu((1, 64, 2, 64)), cpu((1, 64, 2, 64)), v, v, beta)
    with pytest.raises(ValueError, match="divisible"):
        B.chunk_kda(q, q, cpu((1, 64, 3, 128)), cpu((1, 64, 3, 128)), cpu((1, 64, 3)))
    with pytest.raises(ValueError, match="beta"):
        B.chunk_kda(q, q, v, v, cpu((1, 64, 2)))
    with pytest.raises(TypeError):
        B.chunk_kda(q.double(), q.double(), v.double(), v.double(), beta.double())
    with pytest.raises(TypeError):
        B.chunk_kda(q, q, v.float(), v, beta)
    with pytest.raises(ValueError, match="4D"):
        B.chunk_kda(q[0], q[0], v[0], v[0], beta[0])
    cu = torch.tensor([0, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="varlen"):
        B.chunk_kda(torch.cat([q, q]), torch.cat([q, q]), torch.cat([v, v]),
                    torch.cat([v, v]), torch.cat([beta, beta]), cu_seqlens=cu)
    with pytest.raises(TypeError, match="cu_seqlens"):
        B.chunk_kda(q, q, v, v, beta, cu_seqlens=cu.float())
    with pytest.raises(ValueError, match="state_cache replaces"):
        B.chunk_kda(q, q, v, v, beta, cu_seqlens=cu, state_cache=cpu((2, 4, 128, 128),
                    torch.float32), initial_state=cpu((1, 4, 128, 128), torch.float32))


def test_binding_decode_checks():
    q = cpu((4, 2, 128))
    v = cpu((4, 4, 128))
    cache = cpu((8, 4, 128, 128), torch.float32)
    with pytest.raises(ValueError, match="divisible"):
        B.kda_decode(q, q, cpu((4, 3, 128)), cpu((4, 3, 128)), cpu((4, 3)), cache)
    # two tokens per request need [N, T] state indices; more than 8 are not served
    with pytest.raises(ValueError, match="state_indices"):
        B.kda_decode(cpu((4, 2, 2, 128)), cpu((4, 2, 2, 128)), cpu((4, 2, 4, 128)),
                     cpu((4, 2, 4, 128)), cpu((4, 2, 4)), cache)
    with pytest.raises(ValueError, match="columns"):
        B.kda_decode(cpu((4, 2, 2, 128)), cpu((4, 2, 2, 128)), cpu((4, 2, 4, 128)),
                     cpu((4, 2, 4, 128)), cpu((4, 2, 4)), cache,
                     torch.zeros((4, 1), dtype=torch.int32))
    with pytest.raises(NotImplementedError):
        B.kda_decode(cpu((4, 9, 2, 128)), cpu((4, 9, 2, 128)), cpu((4, 9, 4, 128)),
                     cpu((4, 9, 4, 128)), cpu((4, 9, 4)), cache)
    with pytest.raises(ValueError, match="single-token"):
        B.kda_decode(q, q, v, v, cpu((4, 4)), cache, torch.zeros(4, dtype=torch.int32),
                     num_accepted_tokens=torch.ones(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="pool"):
        B.kda_decode(q, q, v, v, cpu((4, 4)), cpu((8, 4, 128, 64), torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        B.kda_decode(q, q, v, v, cpu((4, 4)), cache.half())


def test_planner_picks_groups_only_for_long_chains(lib):
    """Workspace grows by the scan planes exactly when the planner groups
    (staged walk planner)."""
    def total(**kw):
        a = chunk_args(path=B.PATH_FUSED, **kw)
        lay = B.WsLayout()
        assert lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay)) == B.KDA_OK
        return lay.total - lay.scan
    # 4 x 4096 tokens over 16 heads: 256 two-wave workgroups of 64-chunk
    # chains fill the device -> no scan
    assert total(num_seqs=4, total_tokens=4 * 4096, hqk=16, hv=16) == 0
    # one 131072-token sequence over 32 heads: 2048-chunk chains -> scan planes
    assert total(num_seqs=1, total_tokens=131072, hqk=32, hv=32) > 0
    # explicit groups always reserve their planes
    assert total(num_seqs=2, total_tokens=256, groups=4) == 4 * 2 * 4 * 3 * 128 * 128 * 4


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: the checks fail first


@pytest.mark.parametrize("make,call", [
    (chunk_args, lambda lib, a: ws_size(lib, a)[0]),
    (decode_args, lambda lib, a: lib.kda_decode(ctypes.byref(a))),
], ids=["chunk", "decode"])
@pytest.mark.parametrize("fields,status", [
    (dict(A_log=FAKE), B.KDA_ERR_SHAPE),                       # without dt_bias
    (dict(dt_bias=FAKE), B.KDA_ERR_SHAPE),                     # without A_log
    (dict(A_log=FAKE, dt_bias=FAKE, dt_bias_dtype=2, lower_bound=-5.0), B.KDA_ERR_DTYPE),
    (dict(A_log=FAKE, dt_bias=FAKE, dt_bias_dtype=0, lower_bound=-11.0), B.KDA_ERR_UNSUPPORTED),
    (dict(A_log=FAKE, dt_bias=FAKE, dt_bias_dtype=0, lower_bound=-5.01), B.KDA_ERR_UNSUPPORTED),
    (dict(A_log=FAKE, dt_bias=FAKE, dt_bias_dtype=0, lower_bound=0.5), B.KDA_ERR_UNSUPPORTED),
    (dict(A_log=FAKE, dt_bias=FAKE, dt_bias_dtype=1, lower_bound=float("nan")),
     B.KDA_ERR_UNSUPPORTED),
], ids=["a_only", "bias_only", "bias_f16", "lb_low", "lb_below_5", "lb_pos", "lb_nan"])
def test_gate_parameter_checks(lib, make, call, fields, status):
    a = make(**fields)
    assert call(lib, a) == status
    assert lib.kda_last_error().decode() != ""


def test_binding_gate_checks():
    q = cpu((1, 64, 2, 128))
    v = cpu((1, 64, 4, 128))
    beta = cpu((1, 64, 4))
    a_log = torch.zeros(4)
    with pytest.raises(ValueError, match="together"):
        B.chunk_kda(q, q, v, v, beta, A_log=a_log)
    with pytest.raises(ValueError, match="shape"):
        B.chunk_kda(q, q, v, v, beta, A_log=a_log, dt_bias=torch.zeros(4, 64))
    with pytest.raises(TypeError):
        B.chunk_kda(q, q, v, v, beta, A_log=a_log.double(), dt_bias=torch.zeros(4, 128))
    with pytest.raises(TypeError):
        B.chunk_kda(q, q, v, v, beta, A_log=a_log, dt_bias=torch.zeros(4, 128).half())


@pytest.mark.parametrize("fields,status", [
    (dict(checkpoint_state=FAKE), B.KDA_ERR_SHAPE),                      # no offsets
    (dict(checkpoint_offsets=FAKE), B.KDA_ERR_SHAPE),                    # no state
    (dict(checkpoint_state=FAKE, checkpoint_offsets=FAKE, checkpoint_rows=0), B.KDA_ERR_SHAPE),
    (dict(checkpoint_state=FAKE, checkpoint_offsets=FAKE, checkpoint_rows=1), B.KDA_ERR_SHAPE),
], ids=["state_only", "offsets_only", "no_rows", "row_per_seq"])
def test_checkpoint_argument_checks(lib, fields, status):
    a = chunk_args(**fields)   # 2 sequences
    assert ws_size(lib, a)[0] == status


def test_checkpoint_rows_with_indices_pass_checks(lib):
    a = chunk_args(checkpoint_state=FAKE, checkpoint_offsets=FAKE, checkpoint_state_indices=FAKE,
                   checkpoint_rows=1)
    assert ws_size(lib, a)[0] == B.KDA_OK



@pytest.mark.parametrize("fields,status", [
    (dict(tokens=9, state_index_cols=9, state_indices=FAKE), B.KDA_ERR_UNSUPPORTED),
    (dict(tokens=2), B.KDA_ERR_SHAPE),                                  # needs 2-D indices
    (dict(tokens=4, state_index_cols=3, state_indices=FAKE), B.KDA_ERR_SHAPE),
    (dict(state_index_cols=2), B.KDA_ERR_SHAPE),                        # cols without indices
    (dict(num_accepted_tokens=FAKE, state_indices=FAKE), B.KDA_ERR_SHAPE),  # 1-D with counts
], ids=["t9", "t2_1d", "cols_short", "cols_no_idx", "acc_1d"])
def test_multi_token_decode_checks(lib, fields, status):
    a = decode_args(**fields)
    assert lib.kda_decode(ctypes.byref(a)) == status



def test_state_dtype_checks(lib):
    # chunk: the states (dense or paged) are fp32 or of the input dtype, never fp16
    assert ws_size(lib, chunk_args(state_dtype=2))[0] == B.KDA_ERR_DTYPE   # f16 with bf16 input
    assert ws_size(lib, chunk_args(state_dtype=1))[0] == B.KDA_OK
    a = chunk_args(state_dtype=1, state_cache=FAKE, state_indices=FAKE, has_initial_state=FAKE,
                   num_slots=4)
    assert ws_size(lib, a)[0] == B.KDA_OK                                  # bf16 pool
    a = chunk_args(dtype=0, state_dtype=1, state_cache=FAKE, state_indices=FAKE,
                   has_initial_state=FAKE, num_slots=4)
    assert ws_size(lib, a)[0] == B.KDA_ERR_DTYPE                           # bf16 pool, fp32 in
    assert ws_size(lib, chunk_args(dtype=2))[0] == B.KDA_OK                # fp16 inputs
    assert ws_size(lib, chunk_args(dtype=2, state_dtype=2))[0] == B.KDA_ERR_UNSUPPORTED
    assert ws_size(lib, chunk_args(dtype=2, path=B.PATH_ONCHIP))[0] == B.KDA_ERR_UNSUPPORTED
    # fp16 inputs keep fp32 intermediates: the same layout as fp32 inputs
    l16, l32 = B.WsLayout(), B.WsLayout()
    assert lib.kda_chunk_ws_layout(ctypes.byref(chunk_args(dtype=2)), ctypes.byref(l16)) == B.KDA_OK
    assert lib.kda_chunk_ws_layout(ctypes.byref(chunk_args(dtype=0)), ctypes.byref(l32)) == B.KDA_OK
    assert l16.total == l32.total and l16.aqk == l32.aqk
    # decode: fp32 or bf16 cache
    assert lib.kda_decode(ctypes.byref(decode_args(state_dtype=2))) == B.KDA_ERR_DTYPE


def test_binding_state_dtype_rules():
    q = cpu((1, 64, 2, 128))
    v = cpu((1, 64, 4, 128))
    beta = cpu((1, 64, 4))
    with pytest.raises(TypeError, match="initial_state"):
        B.chunk_kda(q, q, v, v, beta, initial_state=cpu((1, 4, 128, 128), torch.float16))
    q16, v16, b16 = q.half(), v.half(), beta.half()
    with pytest.raises(TypeError, match="initial_state"):   # fp16 inputs: fp32 states only
        B.chunk_kda(q16, q16, v16, v16, b16, initial_state=cpu((1, 4, 128, 128), torch.float16))
    with pytest.raises(TypeError, match="state_cache"):
        B.chunk_kda(q16, q16, v16, v16, b16, state_cache=cpu((3, 4, 128, 128), torch.float16),
                    state_indices=torch.zeros(1, dtype=torch.int32),
                    has_initial_state=torch.zeros(1, dtype=torch.uint8))
    with pytest.raises(TypeError, match="same dtype"):
        B.chunk_kda(q, q, v, v, beta, initial_state=cpu((1, 4, 128, 128)),
                    output_final_state=True, final_state=cpu((1, 4, 128, 128), torch.float32))


def test_misaligned_tensor_pointers_are_rejected(lib):
    """Base pointers of the tensors read with vector loads must be 16-byte
    aligned; the check runs before anything touches device memory."""
    odd = ctypes.c_void_p(0x1008)
    for field in ("initial_state", "final_state"):
        assert ws_size(lib, chunk_args(**{field: odd}))[0] == B.KDA_ERR_ARG
    assert lib.kda_decode(ctypes.byref(decode_args(q=odd, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
                                                   out=FAKE, state_cache=FAKE))) == B.KDA_ERR_ARG
    assert lib.kda_decode(ctypes.byref(decode_args(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
                                                   out=FAKE, state_cache=odd))) == B.KDA_ERR_ARG
    # beta is exempt (read one element at a time)
    a = decode_args(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=ctypes.c_void_p(0x1002), out=FAKE,
                    state_cache=odd)
    assert lib.kda_decode(ctypes.byref(a)) == B.KDA_ERR_ARG
    assert b"16-byte" in lib.kda_last_error()


def test_token_stride_of_projection_views():
    """Views into a wider projection output pass their per-token stride; a
    contiguous tensor passes 0; layouts the kernels cannot read are refused."""
    T, W = 10, 3 * 256 + 2 * 512 + 4
    proj = torch.zeros(T, W)
    q = proj[:, :256].view(T, 2, 128)
    g = proj[:, 768:1280].view(T, 4, 128)
    beta = proj[:, W - 4:]
    assert B._token_stride("q", q, 2) == W
    assert B._token_stride("g", g, 2) == W
    assert B._token_stride("beta", beta, 1) == W
    assert B._token_stride("q", q.contiguous(), 2) == 0
    # [B, T, H, 128] with a batch stride of T tokens flattens to one stride
    q4 = proj.view(2, 5, W)[..., :256].view(2, 5, 2, 128)
    assert B._token_stride("q", q4, 2) == W
    with pytest.raises(ValueError, match="fixed stride"):   # channels not contiguous
        B._token_stride("q", torch.zeros(T, 128, 2).transpose(1, 2), 2)
    with pytest.raises(ValueError, match="fixed stride"):   # heads not 128 apart
        B._token_stride("q", torch.zeros(T, 2, 256)[..., :128], 2)
    with pytest.raises(ValueError, match="fixed stride"):   # tokens not one stride apart
        B._token_stride("q", torch.zeros(4, 8, 2, 128)[:, :5], 2)
    pool = torch.zeros(3, 2 * 128 * 128 + 64)
    cache = pool[:, :2 * 128 * 128].view(3, 2, 128, 128)
    assert B._slot_stride(cache) == 2 * 128 * 128 + 64
    assert B._slot_stride(cache.contiguous()) == 0
    with pytest.raises(ValueError, match="dense"):
        B._slot_stride(torch.zeros(3, 2, 128, 128).transpose(2, 3))


def test_stride_checks(lib):
    # chunk_args: hqk = 2, hv = 4, bf16
    assert ws_size(lib, chunk_args(q_stride=256))[0] == B.KDA_OK          # = dense
    assert ws_size(lib, chunk_args(q_stride=1024 + 8))[0] == B.KDA_OK     # 16-byte rows
    assert ws_size(lib, chunk_args(q_stride=255))[0] == B.KDA_ERR_SHAPE   # below dense
    assert ws_size(lib, chunk_args(g_stride=512 + 4))[0] == B.KDA_ERR_ARG  # 8-byte rows
    assert ws_size(lib, chunk_args(beta_stride=3))[0] == B.KDA_ERR_SHAPE
    assert ws_size(lib, chunk_args(beta_stride=4 + 3))[0] == B.KDA_OK     # beta: any stride
    assert ws_size(lib, chunk_args(v_stride=(1 << 24) + 8))[0] == B.KDA_ERR_SHAPE
    assert ws_size(lib, chunk_args(state_slot_stride=4 * 128 * 128))[0] == B.KDA_ERR_SHAPE
    paged = dict(state_cache=FAKE, state_indices=FAKE, has_initial_state=FAKE, num_slots=4)
    assert ws_size(lib, chunk_args(state_slot_stride=4 * 128 * 128 + 8, **paged))[0] == B.KDA_OK
    assert ws_size(lib, chunk_args(state_slot_stride=4 * 128 * 128 - 8,
                                   **paged))[0] == B.KDA_ERR_SHAPE
    assert ws_size(lib, chunk_args(state_slot_stride=4 * 128 * 128 + 4,
                                   **paged))[0] == B.KDA_ERR_SHAPE
    ptrs = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, out=FAKE, state_cache=FAKE)
    assert lib.kda_decode(ctypes.byref(decode_args(q_stride=100, **ptrs))) == B.KDA_ERR_SHAPE
    assert lib.kda_decode(ctypes.byref(decode_args(k_stride=260, **ptrs))) == B.KDA_ERR_ARG
    assert lib.kda_decode(ctypes.byref(decode_args(state_slot_stride=100,
                                                   **ptrs))) == B.KDA_ERR_SHAPE


def test_planner_picks_measured_best_on_the_standard_workloads():
    """Host-only planning (no device work): the dense prefill walks without
    groups on 2-wave workgroups, the varlen GVA batch (768 chains) on 8-wave
    workgroups, and the single long sequence takes the 8-group scan on 8-wave
    ones (each the fastest in a sweep of G and walk widths on MI355X)."""
    from gated_delta_rule_65_amd import inputs

    def plan(wl):
        r = inputs.WORKLOADS[wl]
        hqk, hv, dt = r["hqk"], r["hv"], r["dtype"]
        if r["kind"] == "chunk_paged":
            gen = torch.Generator()
            gen.manual_seed(1)
            lengths = inputs.varlen_lengths(gen, r["S"], r["N"], r["lo"], r["hi"])
            T = sum(lengths)
            q = torch.zeros(T, hqk, 128, dtype=dt)
            v = torch.zeros(T, hv, 128, dtype=dt)
            cu = torch.tensor([0] + torch.tensor(lengths).cumsum(0).tolist(), dtype=torch.int32)
            return B.chunk_plan(q, q, v, v, torch.zeros(T, hv, dtype=dt), cu_seqlens=cu,
                                path=B.PATH_FUSED)
        shp = (r["B"], r["T"])
        q = torch.zeros(*shp, hqk, 128, dtype=dt)
        v = torch.zeros(*shp, hv, 128, dtype=dt)
        return B.chunk_plan(q, q, v, v, torch.zeros(*shp, hv, dtype=dt), path=B.PATH_FUSED)

    assert plan("dense_prefill") == (1, 2)
    assert plan("varlen_gva_paged") == (1, 8)
    assert plan("long_single") == (8, 8)


def test_planner_max_seqlen_hint(lib):
    """The longest sequence bounds a varlen walk.  With host offsets the
    binding passes it as a planning hint; without it the batch is planned as
    if its sequences were equally long, so an equal-length batch given in
    varlen form plans like the dense one."""
    def varlen(lengths, hqk, hv):
        T = sum(lengths)
        q = torch.zeros(T, hqk, 128, dtype=torch.bfloat16)
        v = torch.zeros(T, hv, 128, dtype=torch.bfloat16)
        cu = torch.tensor([0] + torch.tensor(lengths).cumsum(0).tolist(), dtype=torch.int32)
        return q, v, torch.zeros(T, hv, dtype=torch.bfloat16), cu
    F = B.PATH_FUSED
    q, v, beta, cu = varlen([4096] * 4, 16, 16)
    assert B.chunk_plan(q, q, v, v, beta, cu_seqlens=cu, path=F) == (1, 2)
    assert B.chunk_plan(q, q, v, v, beta, cu_seqlens=cu, max_seqlen=0, path=F) == (1, 2)
    # one long sequence among short ones: the hint moves the plan
    q, v, beta, cu = varlen([8192] + [128] * 60, 4, 16)
    with_hint = B.chunk_plan(q, q, v, v, beta, cu_seqlens=cu, path=F)
    without = B.chunk_plan(q, q, v, v, beta, cu_seqlens=cu, max_seqlen=0, path=F)
    assert with_hint != without
    assert ws_size(lib, chunk_args(max_seqlen=-1))[0] == B.KDA_ERR_SHAPE


# ------------------------------------------------- verify window and commit

def verify_args(**kw):
    a = B.VerifyArgs()
    a.struct_size = ctypes.sizeof(B.VerifyArgs)
    a.dtype, a.n, a.hqk, a.hv, a.window = 1, 4, 2, 4, 4
    a.scale, a.use_qk_l2norm, a.num_slots, a.lower_bound = 0.1, 1, 8, -5.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def commit_args(**kw):
    a = B.CommitArgs()
    a.struct_size = ctypes.sizeof(B.CommitArgs)
    a.dtype, a.n, a.hv, a.window, a.num_slots, a.use_qk_l2norm = 1, 4, 4, 4, 8, 1
    a.lower_bound = -5.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_struct_layouts_match_the_header(tmp_path):
    """Every field offset of the ctypes mirrors equals the C header's (gcc)."""
    structs = {"kda_chunk_args": B.ChunkArgs, "kda_decode_args": B.DecodeArgs,
               "kda_verify_args": B.VerifyArgs, "kda_commit_args": B.CommitArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kda.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    want = {}
    for cname, py in structs.items():
        want[f"{cname} size"] = ctypes.sizeof(py)
        for f, _ in py._fields_:
            want[f"{cname} {f}"] = getattr(py, f).offset
    for line in filter(None, got):
        key, val = line.rsplit(" ", 1)
        assert want[key] == int(val), line


@pytest.mark.parametrize("field,value,status", [
    ("hv", 3, B.KDA_ERR_SHAPE),
    ("dtype", 5, B.KDA_ERR_DTYPE),
    ("n", -1, B.KDA_ERR_SHAPE),
    ("window", 0, B.KDA_ERR_SHAPE),
    ("window", 9, B.KDA_ERR_SHAPE),
    ("num_slots", 0, B.KDA_ERR_SHAPE),
    ("state_dtype", 2, B.KDA_ERR_DTYPE),
    ("struct_size", 8, B.KDA_ERR_ARG),
    ("state_slot_stride", 100, B.KDA_ERR_SHAPE),
    ("q_stride", 8, B.KDA_ERR_SHAPE),
])
def test_verify_checks(lib, field, value, status):
    assert lib.kda_verify(ctypes.byref(verify_args(**{field: value}))) == status


@pytest.mark.parametrize("field,value,status", [
    ("hv", 0, B.KDA_ERR_SHAPE),
    ("dtype", 5, B.KDA_ERR_DTYPE),
    ("n", -1, B.KDA_ERR_SHAPE),
    ("window", 9, B.KDA_ERR_SHAPE),
    ("num_slots", 0, B.KDA_ERR_SHAPE),
    ("state_dtype", 2, B.KDA_ERR_DTYPE),
    ("struct_size", 8, B.KDA_ERR_ARG),
])
def test_commit_checks(lib, field, value, status):
    assert lib.kda_commit(ctypes.byref(commit_args(**{field: value}))) == status


def test_verify_and_commit_null_pointers_gate_and_empty_batch(lib):
    # n > 0 with NULL tensors: rejected before any launch
    assert lib.kda_verify(ctypes.byref(verify_args())) == B.KDA_ERR_ARG
    assert lib.kda_commit(ctypes.byref(commit_args())) == B.KDA_ERR_ARG
    # gate parameters: both or neither, lower_bound in [-5, 0]
    one = ctypes.c_float(0.0)
    assert lib.kda_verify(ctypes.byref(verify_args(A_log=ctypes.addressof(one)))) == \
        B.KDA_ERR_SHAPE
    assert lib.kda_commit(ctypes.byref(commit_args(
        A_log=ctypes.addressof(one), dt_bias=ctypes.addressof(one), lower_bound=-6.0))) == \
        B.KDA_ERR_UNSUPPORTED
    # an empty batch is a no-op
    assert lib.kda_verify(ctypes.byref(verify_args(n=0))) == B.KDA_OK
    assert lib.kda_commit(ctypes.byref(commit_args(n=0))) == B.KDA_OK


def test_binding_verify_and_commit_checks():
    q = torch.zeros(5, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(5, 4, 128, dtype=torch.bfloat16)
    beta = torch.zeros(5, 4, dtype=torch.bfloat16)
    cache = torch.zeros(3, 4, 128, 128)
    qs = torch.tensor([0, 2, 5])
    idx = torch.tensor([0, 1])
    with pytest.raises(ValueError):   # window past 8
        B.kda_verify(q, q, v, v, beta, qs, cache, idx, 9)
    with pytest.raises(ValueError):   # Hv not a multiple of Hqk
        B.kda_verify(q[:, :1].expand(5, 3, 128), q[:, :1].expand(5, 3, 128), v, v, beta,
                     qs, cache, idx, 4)
    with pytest.raises(TypeError):    # mixed dtypes
        B.kda_verify(q, q.float(), v, v, beta, qs, cache, idx, 4)
    with pytest.raises(ValueError):   # state_indices shape
        B.kda_verify(q, q, v, v, beta, qs, cache, torch.tensor([0]), 4)
    with pytest.raises(ValueError):   # pool of the wrong head count
        B.kda_verify(q, q, v, v, beta, qs, cache[:, :2], idx, 4)
    corr = torch.zeros(2, 4, 4, 128)
    kg = torch.zeros(2, 4, 4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # corr must be fp32
        B.kda_commit(cache, idx, torch.tensor([1, 2]), corr.double(), kg)
    with pytest.raises(ValueError):   # kg shape
        B.kda_commit(cache, idx, torch.tensor([1, 2]), corr, kg[:, :, :3])
    with pytest.raises(ValueError):   # accepted counts shape
        B.kda_commit(cache, idx, torch.tensor([1]), corr, kg)


def test_build_rejects_kernels_that_spill():
    """The build parses the compiler's resource remarks and fails on any kernel
    with private scratch (a register spill)."""
    from gated_delta_rule_65_amd import build
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._spilling_kernels(remarks) == [("kern_b", 12)]


LOG_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
from gated_delta_rule_65_amd import binding as B
lib = B.load_library()
a = B.ChunkArgs()
a.struct_size = ctypes.sizeof(B.ChunkArgs)
a.dtype, a.num_seqs, a.total_tokens, a.hqk, a.hv = 1, 0, 0, 2, 4
a.scale, a.use_qk_l2norm = 128 ** -0.5, 1
fake = ctypes.c_void_p(0x1000)
for f in ("q", "k", "v", "g", "beta", "out"):
    setattr(a, f, fake)
n = ctypes.c_size_t(0)
assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
a.workspace, a.workspace_bytes = fake, n.value
sys.exit(lib.kda_chunk_fwd(ctypes.byref(a)))   # empty batch: nothing is queued
"""


@pytest.mark.parametrize("value", ["1", None])
def test_kda_log_prints_the_launch_plan(value):
    env = dict(os.environ)
    env.pop("KDA_LOG", None)
    if value is not None:
        env["KDA_LOG"] = value
    r = subprocess.run(["python", "-c", LOG_SCRIPT.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("kda: ")]
    if value is None:
        assert lines == []
    else:
        assert len(lines) == 1, r.stderr
        for field in ("chunk_fwd", "path=fused", "groups=1", "walk_waves=", "BV=",
                      "walk_wgs=", "workspace="):
            assert field in lines[0], lines[0]
