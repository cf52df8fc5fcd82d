"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.
No call here reaches a kernel (every case fails validation, or has N = 0)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_97_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
BF16, F32 = kda.KDA_DTYPE_BF16, kda.KDA_DTYPE_F32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kda_chunk_prefill", "kda_decode_step", "kda_chunk_prefill_workspace_size",
            "kda_status_string"} <= set(names)
    lib = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kda.h but not exported"


def test_status_strings():
    for code in range(0, -10, -1):
        s = kda.kda_status_string(code)
        assert s and s != "unknown status"
    assert kda.kda_status_string(-99) == "unknown status"


def test_workspace_size():
    w1 = kda.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 1, 64, BF16)
    # W, q e^Gam, K~^T, Ut (bf16), the scores P in 16 x 32 blocks up to each
    # 16-row tile's diagonal (1 + 1 + 2 + 2 blocks, bf16) and the decay (fp32)
    # per (chunk, head), plus the chunk map
    slots = (8192 // 64 + 1) * 32
    per_slot = 4 * 64 * 128 * 2 + 6 * 16 * 32 * 2 + 128 * 4
    # this call runs as two chunk windows: plus the carried fp32 state
    carry = 32 * 128 * 128 * 4
    assert slots * per_slot + carry <= w1 < slots * per_slot + carry + (1 << 20)
    assert w1 % 256 == 0
    w2 = kda.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 64, 64, BF16)
    assert w2 > w1
    assert kda.kda_chunk_prefill_workspace_size(4, 100, 2, 32, 32, 4, 16, F32) > 0
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_workspace_size(1, 100, 2, 48, 32, 1, 64, BF16)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    assert kda.kda_chunk_prefill_workspace_size(1, 100, 2, 128, 128, 1, 64, F32) > 0  # fp32, chunk 64, d = 128
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_workspace_size(1, 100, 2, 64, 64, 1, 32, BF16)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_workspace_size(2, 100, 2, 64, 64, 3, 64, BF16)
    assert e.value.status == kda.KDA_ERR_SHAPE
    # one chunk's output rows must span less than 2 GiB at fp32 width
    assert kda.kda_chunk_prefill_workspace_size(1, 64, 65535, 128, 128, 1, 64, BF16) > 0
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_workspace_size(1, 64, 65536, 128, 128, 1, 64, BF16)
    assert e.value.status == kda.KDA_ERR_SHAPE



def test_workspace_segment_states_follow_the_plan():
    """1M tokens x 8 heads (32 chains of 32 columns, long) runs segment-parallel
    with 32 segments per head: the workspace adds three fp32 dk x dv states per
    (segment, head), the two summaries and the scanned incoming state.  The
    H = 32, T = 8192 call (128 chains) and a sequence under 64 chunks run one
    chain per head and add none; so does a 64-chunk sequence at d = 128, bf16,
    chunk 64, where the loader-fed single chain is faster, while 128 chunks
    of one head take 16 segments of 8."""
    per_slot = 4 * 64 * 128 * 2 + 6 * 16 * 32 * 2 + 128 * 4
    st = 128 * 128 * 4

    def extra(T, H):
        w = kda.kda_chunk_prefill_workspace_size(1, T, H, 128, 128, 1, 64, BF16)
        return w - (T // 64 + 1) * H * per_slot

    assert 3 * 32 * 8 * st <= extra(1 << 20, 8) < 3 * 32 * 8 * st + (1 << 20)
    assert 32 * st <= extra(8192, 32) < 33 * st  # no segments; the chunk-window carry
    assert 0 <= extra(63 * 64, 1) < st
    assert 0 <= extra(64 * 64, 1) < st
    assert 3 * 16 * st <= extra(128 * 64, 1) < 3 * 16 * st + (1 << 20)


def test_workspace_window_carry_follows_the_plan():
    """Fixed-length bf16 batches at d = 128, chunk 64 whose hand-off between the
    passes (72,192 bytes per (chunk, head)) passes 192 MiB run as windows of
    about 160 MiB: groups of whole sequences when a sequence's hand-off fits,
    else windows over each sequence's chunks (at least 32 chunks each) with
    an fp32 carry state per (sequence, head) in the workspace.  Only chunk
    windows add the carry."""
    per_slot = 4 * 64 * 128 * 2 + 6 * 16 * 32 * 2 + 128 * 4
    st = 128 * 128 * 4

    def extra(B, T, H, N=None):
        N = B if N is None else N
        w = kda.kda_chunk_prefill_workspace_size(B, T, H, 128, 128, N, 64, BF16)
        slots = B * T // 64 + (1 if B == 1 else 0)  # B = 1 may also be read as packed: one slot more
        return w - slots * H * per_slot

    assert 32 * st <= extra(1, 8192, 32) < 33 * st   # 282 MiB, one sequence: two chunk windows
    assert 48 * st <= extra(1, 8192, 48) < 49 * st   # 423 MiB: three chunk windows
    assert 64 * st <= extra(1, 8192, 64) < 65 * st   # 564 MiB: four, 32 chunks each
    assert 128 * st <= extra(4, 8192, 32) < 129 * st  # 1.1 GiB: two chunk windows per sequence
    assert extra(2, 4096, 32) < st              # 282 MiB over two sequences: one per window, no carry
    assert extra(2, 4096, 24) < st              # 211 MiB: the same
    assert extra(2, 4096, 16) < st              # 141 MiB: no windows
    assert extra(1, 63 * 64, 32) < st           # 139 MiB over 63 chunks: no windows
    assert extra(1, 3072, 128) < st             # 423 MiB, but 48 chunks: windows of 16 would not pay




# fake, never-dereferenced device addresses (validation fails before use)
A = 1 << 32


def _prefill(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24), h0=0,
                cu_seqlens=0, B=1, T=64, H=2, dk=32, dv=32, num_seqs=1, chunk_size=16, dtype=F32,
                flags=0, o=A + (5 << 24), ht=A + (6 << 24), workspace=A + (7 << 24), workspace_bytes=1 << 20,
                stream=0)
    args.update(kw)
    return kda.kda_chunk_prefill(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk_size=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=7), kda.KDA_ERR_UNSUPPORTED),
    (dict(H=0), kda.KDA_ERR_SHAPE),
    (dict(T=-1), kda.KDA_ERR_SHAPE),
    (dict(num_seqs=2), kda.KDA_ERR_SHAPE),                            # N must equal B without cu_seqlens
    (dict(B=2, num_seqs=2, cu_seqlens=A + (8 << 24)), kda.KDA_ERR_SHAPE),  # packed needs B = 1
    (dict(q=0), kda.KDA_ERR_NULL),
    (dict(g=0), kda.KDA_ERR_NULL),
    (dict(o=0), kda.KDA_ERR_NULL),
    (dict(workspace=0), kda.KDA_ERR_WORKSPACE),
    (dict(workspace_bytes=1024), kda.KDA_ERR_WORKSPACE),
    (dict(k=A + (1 << 24) + 8), kda.KDA_ERR_ALIGN),
    (dict(workspace=A + (7 << 24) + 16), kda.KDA_ERR_ALIGN),
    (dict(o=A + 256), kda.KDA_ERR_ALIAS),                             # o overlaps q
    (dict(h0=A + (9 << 24), ht=A + (9 << 24) + 4096), kda.KDA_ERR_ALIAS),  # partial h0/ht overlap
    (dict(workspace=A + (6 << 24)), kda.KDA_ERR_ALIAS),               # workspace overlaps ht
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status


def test_prefill_nothing_to_do():
    # no sequences: nothing is launched, nothing is touched
    assert _prefill(B=0, num_seqs=0, T=0, q=0, k=0, v=0, g=0, beta=0, o=0, ht=0, workspace=0) == kda.KDA_OK


def _decode(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24),
                state=A + (5 << 24), o=A + (6 << 24), N=4, H=2, dk=128, dv=128, dtype=BF16, flags=0, stream=0)
    args.update(kw)
    return kda.kda_decode_step(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=3), kda.KDA_ERR_UNSUPPORTED),
    (dict(H=0), kda.KDA_ERR_SHAPE),
    (dict(N=-1), kda.KDA_ERR_SHAPE),
    (dict(state=0), kda.KDA_ERR_NULL),
    (dict(o=A + (6 << 24) + 2), kda.KDA_ERR_ALIGN),
    (dict(o=A + (5 << 24) + 1024), kda.KDA_ERR_ALIAS),                # o inside the state
    (dict(state=A + 64), kda.KDA_ERR_ALIAS),                          # state overlaps q
])
def test_decode_validation(kw, status):
    assert _decode(**kw) == status


def test_decode_empty_batch():
    assert _decode(N=0, q=0, k=0, v=0, g=0, beta=0, state=0, o=0) == kda.KDA_OK


def _prefill_ck(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24), h0=0,
                cu_seqlens=0, B=1, T=64, H=2, dk=32, dv=32, num_seqs=1, chunk_size=16, dtype=F32,
                flags=0, o=A + (5 << 24), ht=A + (6 << 24), ckpt=A + (10 << 24), ckpt_stride=32, num_ckpt=2,
                workspace=A + (7 << 24), workspace_bytes=1 << 20, stream=0)
    args.update(kw)
    return kda.kda_chunk_prefill_checkpointed(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(ckpt_stride=0), kda.KDA_ERR_SHAPE),
    (dict(ckpt_stride=24), kda.KDA_ERR_SHAPE),                        # not a multiple of the chunk
    (dict(num_ckpt=-1), kda.KDA_ERR_SHAPE),
    (dict(ckpt=0), kda.KDA_ERR_NULL),
    (dict(ckpt=A + (10 << 24) + 4), kda.KDA_ERR_ALIGN),
    (dict(ckpt=A + (6 << 24) + 1024), kda.KDA_ERR_ALIAS),             # inside ht
    (dict(ckpt=A + 128), kda.KDA_ERR_ALIAS),                          # overlaps q
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),                           # the prefill's own checks still apply
    (dict(q=0), kda.KDA_ERR_NULL),
])
def test_prefill_checkpointed_validation(kw, status):
    assert _prefill_ck(**kw) == status


def test_prefill_checkpointed_no_slots_and_nothing_to_do():
    assert _prefill_ck(B=0, num_seqs=0, T=0, q=0, k=0, v=0, g=0, beta=0, o=0, ht=0, workspace=0, ckpt=0,
                       num_ckpt=0) == kda.KDA_OK


def test_checkpoint_count():
    assert kda.checkpoint_count(700, 128, B=2) == 10
    assert kda.checkpoint_count(0, 128, seqlens=[37, 0, 512, 129, 300]) == 0 + 0 + 4 + 1 + 2


def _verify(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24),
                state=A + (5 << 24), o=A + (6 << 24), N=4, K=3, H=2, dk=128, dv=128, dtype=BF16, flags=0,
                stream=0)
    args.update(kw)
    return kda.kda_decode_verify(**args)


def _commit(**kw):
    args = dict(k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24), n_accept=A + (7 << 24),
                state=A + (5 << 24), N=4, K=3, H=2, dk=128, dv=128, dtype=BF16, flags=0, stream=0)
    args.update(kw)
    return kda.kda_decode_commit(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=3), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=-1), kda.KDA_ERR_SHAPE),
    (dict(H=0), kda.KDA_ERR_SHAPE),
    (dict(o=0), kda.KDA_ERR_NULL),
    (dict(state=0), kda.KDA_ERR_NULL),
    (dict(o=A + (6 << 24) + 2), kda.KDA_ERR_ALIGN),
    (dict(o=A + (5 << 24) + 4096), kda.KDA_ERR_ALIAS),                # o inside the state
    (dict(o=A + 256), kda.KDA_ERR_ALIAS),                             # o overlaps q
])
def test_verify_validation(kw, status):
    assert _verify(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dv=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(N=-1), kda.KDA_ERR_SHAPE),
    (dict(n_accept=0), kda.KDA_ERR_NULL),
    (dict(state=A + (5 << 24) + 8), kda.KDA_ERR_ALIGN),
    (dict(n_accept=A + (7 << 24) + 2), kda.KDA_ERR_ALIGN),
    (dict(state=A + (1 << 24) + 1024), kda.KDA_ERR_ALIAS),            # state overlaps k
])
def test_commit_validation(kw, status):
    assert _commit(**kw) == status


def _verify_keep(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24),
                state=A + (5 << 24), o=A + (6 << 24), u=A + (8 << 24), N=4, K=3, H=2, dk=128, dv=128, dtype=BF16,
                flags=0, stream=0)
    args.update(kw)
    return kda.kda_decode_verify_keep(**args)


def _commit_kept(**kw):
    args = dict(k=A + (1 << 24), g=A + (3 << 24), u=A + (8 << 24), n_accept=A + (7 << 24), state=A + (5 << 24),
                N=4, K=3, H=2, dk=128, dv=128, dtype=BF16, flags=0, stream=0)
    args.update(kw)
    return kda.kda_decode_commit_kept(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dv=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(u=0), kda.KDA_ERR_NULL),
    (dict(o=0), kda.KDA_ERR_NULL),
    (dict(u=A + (8 << 24) + 4), kda.KDA_ERR_ALIGN),
    (dict(u=A + (5 << 24) + 4096), kda.KDA_ERR_ALIAS),                # u inside the state
    (dict(u=A + (6 << 24) + 512), kda.KDA_ERR_ALIAS),                 # u overlaps o
    (dict(u=A + 256), kda.KDA_ERR_ALIAS),                             # u overlaps q
])
def test_verify_keep_validation(kw, status):
    assert _verify_keep(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dk=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=-1), kda.KDA_ERR_SHAPE),
    (dict(u=0), kda.KDA_ERR_NULL),
    (dict(n_accept=0), kda.KDA_ERR_NULL),
    (dict(u=A + (8 << 24) + 8), kda.KDA_ERR_ALIGN),
    (dict(n_accept=A + (7 << 24) + 2), kda.KDA_ERR_ALIGN),
    (dict(state=A + (8 << 24) + 1024), kda.KDA_ERR_ALIAS),            # state overlaps u
    (dict(state=A + (3 << 24) + 1024), kda.KDA_ERR_ALIAS),            # state overlaps g
])
def test_commit_kept_validation(kw, status):
    assert _commit_kept(**kw) == status


def _commit_verify(**kw):
    args = dict(prev_k=A + (1 << 24), prev_g=A + (3 << 24), prev_u=A + (8 << 24), n_accept=A + (7 << 24), Kp=3,
                q=A + (9 << 24), k=A + (10 << 24), v=A + (11 << 24), g=A + (12 << 24), beta=A + (13 << 24),
                state=A + (5 << 24), o=A + (6 << 24), u=A + (14 << 24), N=4, K=3, H=2, dk=128, dv=128, dtype=BF16,
                flags=0, stream=0)
    args.update(kw)
    return kda.kda_decode_commit_verify(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(Kp=-1), kda.KDA_ERR_SHAPE),
    (dict(prev_u=0), kda.KDA_ERR_NULL),                              # a previous round needs its kept u
    (dict(n_accept=0), kda.KDA_ERR_NULL),
    (dict(q=0), kda.KDA_ERR_NULL),
    (dict(state=0), kda.KDA_ERR_NULL),
    (dict(prev_u=A + (8 << 24) + 4), kda.KDA_ERR_ALIGN),
    (dict(n_accept=A + (7 << 24) + 2), kda.KDA_ERR_ALIGN),
    (dict(u=A + (5 << 24) + 4096), kda.KDA_ERR_ALIAS),               # new u inside the state
    (dict(state=A + (8 << 24) + 1024), kda.KDA_ERR_ALIAS),           # state overlaps the kept u
    (dict(o=A + (9 << 24) + 512), kda.KDA_ERR_ALIAS),                # o overlaps q
])
def test_commit_verify_validation(kw, status):
    assert _commit_verify(**kw) == status


def test_commit_verify_optional_parts():
    # nothing to commit (Kp = 0, no previous buffers) and nothing to verify (K = 0, no draft buffers)
    assert _commit_verify(N=0) == kda.KDA_OK
    assert _commit_verify(Kp=0, K=0, prev_k=0, prev_g=0, prev_u=0, n_accept=0, q=0, k=0, v=0, g=0, beta=0, o=0,
                          u=0) == kda.KDA_OK


def test_verify_commit_empty():
    assert _verify(N=0, q=0, k=0, v=0, g=0, beta=0, state=0, o=0) == kda.KDA_OK
    assert _verify(K=0, q=0, k=0, v=0, g=0, beta=0, state=0, o=0) == kda.KDA_OK
    assert _commit(N=0, k=0, v=0, g=0, beta=0, n_accept=0, state=0) == kda.KDA_OK
    assert _verify_keep(K=0, q=0, k=0, v=0, g=0, beta=0, state=0, o=0, u=0) == kda.KDA_OK
    assert _commit_kept(N=0, k=0, g=0, u=0, n_accept=0, state=0) == kda.KDA_OK


def _noalloc(**kw):
    args = dict(q=A, k=A + (1 << 24), v=A + (2 << 24), g=A + (3 << 24), beta=A + (4 << 24), h0=0,
                cu_seqlens=0, B=1, T=64, H=2, dk=32, dv=32, num_seqs=1, chunk_size=16, dtype=F32,
                flags=0, o=A + (5 << 24), ht=A + (6 << 24), stream=0)
    args.update(kw)
    return kda.kda_chunk_prefill_noalloc(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk_size=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(H=0), kda.KDA_ERR_SHAPE),
    (dict(num_seqs=2), kda.KDA_ERR_SHAPE),
    # the headline prefill (H=32, T=8192, d=128) needs ~300 MB of workspace
    (dict(T=8192, H=32, dk=128, dv=128, chunk_size=64, dtype=BF16), kda.KDA_ERR_TOO_LARGE),
    (dict(B=4, num_seqs=4, T=4096, H=16, dk=128, dv=128, chunk_size=64, dtype=BF16), kda.KDA_ERR_TOO_LARGE),
])
def test_noalloc_validation(kw, status):
    """Shape errors and sizes beyond the static scratch are refused on the
    host, before the device (or its scratch array) is touched."""
    assert _noalloc(**kw) == status


def test_noalloc_limit_matches_the_workspace_size():
    lim = kda.NOALLOC_SCRATCH_BYTES
    assert kda.kda_chunk_prefill_workspace_size(1, 2048, 32, 128, 128, 1, 64, BF16) <= lim
    assert kda.kda_chunk_prefill_workspace_size(1, 4096, 32, 128, 128, 1, 64, BF16) > lim



# The Python binding checks every tensor against the sizes it passes to the
# library before anything reaches the device (host tensors suffice: the shape
# check comes first, so a mismatch raises ValueError, never a device call).
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float32)


def test_binding_rejects_mismatched_prefill_tensors():
    import torch
    B, T, H, dk, dv = 1, 70, 2, 64, 32
    q = _t(B, T, H, dk, dtype=torch.bfloat16)
    good = dict(k=_t(B, T, H, dk, dtype=torch.bfloat16), v=_t(B, T, H, dv, dtype=torch.bfloat16),
                g=_t(B, T, H, dk), beta=_t(B, T, H), h0=_t(B, H, dk, dv))
    bad = [("k", _t(B, T - 1, H, dk, dtype=torch.bfloat16)), ("g", _t(B, T, H, dv)), ("beta", _t(B, T, H, 1)),
           ("h0", _t(B, H, dv, dk))]
    for name, t in bad:
        a = dict(good, **{name: t})
        with pytest.raises(ValueError, match=f"^{name} has shape"):
            kda.chunk_prefill(q, a["k"], a["v"], a["g"], a["beta"], a["h0"])
    for name, t in [("o", _t(B, T, H, dk, dtype=torch.bfloat16)), ("ht", _t(2, H, dk, dv)),
                    ("ckpt", _t(3, H, dv, dk))]:
        with pytest.raises(ValueError, match=f"^{name} has shape"):
            kda.chunk_prefill(q, *good.values(), **{name: t}, **({"ckpt_stride": 64} if name == "ckpt" else {}))


def test_binding_rejects_mismatched_decode_tensors():
    import torch
    N, K, H, dk, dv = 3, 4, 2, 64, 32
    bf = torch.bfloat16
    q1, k1, v1 = _t(N, H, dk, dtype=bf), _t(N, H, dk, dtype=bf), _t(N, H, dv, dtype=bf)
    st = _t(N, H, dk, dv)
    with pytest.raises(ValueError, match="^state has shape"):
        kda.decode_step(q1, k1, v1, _t(N, H, dk), _t(N, H), _t(N, H, dv, dk))
    with pytest.raises(ValueError, match="^beta has shape"):
        kda.decode_step(q1, k1, v1, _t(N, H, dk), _t(N, 1), st)
    q, k, v, g, b = _t(N, K, H, dk, dtype=bf), _t(N, K, H, dk, dtype=bf), _t(N, K, H, dv, dtype=bf), \
        _t(N, K, H, dk), _t(N, K, H)
    with pytest.raises(ValueError, match="^v has shape"):
        kda.decode_verify(q, k, _t(N, K - 1, H, dv, dtype=bf), g, b, st)
    with pytest.raises(ValueError, match="^u has shape"):
        kda.decode_verify(q, k, v, g, b, st, u=_t(N, K, H, dk))
    acc = torch.zeros(N, dtype=torch.int32)
    with pytest.raises(ValueError, match="^n_accept has shape"):
        kda.decode_commit(k, v, g, b, torch.zeros(N + 1, dtype=torch.int32), st)
    with pytest.raises(ValueError, match="^u has shape"):
        kda.decode_commit(k, None, g, None, acc, st, u=_t(N, K + 1, H, dv))
    prev = (k, g, _t(N, K, H, dv), acc)
    with pytest.raises(ValueError, match="^prev u has shape"):
        kda.decode_commit_verify((k, g, _t(N, K, H, dk), acc), q, k, v, g, b, st)
    with pytest.raises(ValueError, match="^prev g has shape"):
        kda.decode_commit_verify((k, _t(N, K - 1, H, dk), prev[2], acc), q, k, v, g, b, st)
    with pytest.raises(ValueError, match="^o has shape"):
        kda.decode_commit_verify(prev, q, k, v, g, b, st, o=_t(N, K, H, dk, dtype=bf))
