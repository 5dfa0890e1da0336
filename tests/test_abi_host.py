"""Host-only checks of the C ABI: the library loads, exports every function the header
declares, its NF4 table equals the oracle's bit for bit, and argument validation rejects
bad calls with the documented codes before touching the GPU."""
import ctypes

import numpy as np
import pytest

from lora_fine_tuning_nf4_amd import lnf4
from oracle import nf4 as onf4


@pytest.fixture(scope="module")
def L():
    return lnf4.lib()


def test_exports_every_header_symbol(L):
    names = lnf4.header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n


def test_table_matches_oracle_bitwise(L):
    lib_tab = np.array(lnf4.lnf4_nf4_table(), np.float32)
    assert np.array_equal(lib_tab.view(np.uint32), onf4.nf4_table().view(np.uint32))


def _rc(fn, *args):
    return fn(*args)


FAKE = 1 << 20  # a 16-byte aligned non-NULL address that is never dereferenced


def test_dequant_validation(L):
    assert L.nf4_dequant(FAKE, FAKE, 64, 32, FAKE, None) == lnf4.LNF4_ESHAPE
    assert L.nf4_dequant(FAKE, FAKE, 63, 64, FAKE, None) == lnf4.LNF4_ESHAPE
    assert L.nf4_dequant(None, FAKE, 64, 64, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.nf4_dequant(FAKE + 1, FAKE, 64, 64, FAKE, None) == lnf4.LNF4_EALIGN
    assert L.nf4_dequant(None, None, 0, 64, None, None) == lnf4.LNF4_OK  # empty is a no-op
    assert "blocksize" in lnf4.lnf4_last_error() or lnf4.lnf4_last_error() != ""


def _weight(fmt=0, data=FAKE, absmax=FAKE, out_f=128, in_f=128, bs=64):
    return lnf4.lnf4_weight(fmt, data, absmax, out_f, in_f, bs)


def test_fwd_validation(L):
    fwd = L.lora_linear_fwd
    W = _weight()
    assert fwd(None, FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EINVAL
    assert fwd(ctypes.byref(_weight(in_f=100)), FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_ESHAPE
    assert fwd(ctypes.byref(_weight(bs=32)), FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_ESHAPE
    assert fwd(ctypes.byref(_weight(fmt=7)), FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EINVAL
    assert fwd(ctypes.byref(_weight(absmax=None)), FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EINVAL
    assert fwd(ctypes.byref(_weight(data=FAKE + 2)), FAKE, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EALIGN
    assert fwd(ctypes.byref(W), FAKE, 4, FAKE, FAKE, 65, 1.0, FAKE, FAKE, None) == lnf4.LNF4_EINVAL   # r > 64
    assert fwd(ctypes.byref(W), FAKE, 4, FAKE, None, 8, 1.0, FAKE, FAKE, None) == lnf4.LNF4_EINVAL   # one of A, B
    assert fwd(ctypes.byref(W), FAKE, 4, FAKE, FAKE, 8, 1.0, FAKE, None, None) == lnf4.LNF4_EINVAL   # u missing
    assert fwd(ctypes.byref(W), None, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EINVAL   # x missing
    assert fwd(ctypes.byref(W), FAKE + 8, 4, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EALIGN
    assert fwd(ctypes.byref(W), FAKE, -1, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_EINVAL
    # T = 0 is a no-op that never touches the device
    assert fwd(ctypes.byref(W), None, 0, None, None, 0, 0.0, None, None, None) == lnf4.LNF4_OK


def test_bwd_validation_and_workspace(L):
    W = _weight(out_f=100)
    bwd = L.lora_linear_bwd
    # out_f must be a multiple of 8 in backward
    assert bwd(ctypes.byref(W), FAKE, FAKE, 4, None, None, 0, 0.0, None, FAKE, None, None, 0, None, 0, None) \
        == lnf4.LNF4_ESHAPE
    W = _weight()
    ws = lnf4.lora_linear_bwd_workspace(256, 128, 128, 8)
    assert ws > 0 and ws % 256 == 0
    assert lnf4.lora_linear_bwd_workspace(256, 128, 128, 0) == 0
    # workspace too small
    assert bwd(ctypes.byref(W), FAKE, FAKE, 256, FAKE, FAKE, 8, 1.0, None, FAKE, FAKE, FAKE, 0, FAKE, ws - 256,
               None) == lnf4.LNF4_ESHAPE
    assert bwd(ctypes.byref(W), FAKE, FAKE, 256, FAKE, FAKE, 8, 1.0, None, FAKE, FAKE, FAKE, 0, None, ws,
               None) == lnf4.LNF4_EINVAL
    assert bwd(ctypes.byref(W), FAKE, None, 256, None, None, 0, 0.0, None, FAKE, None, None, 0, None, 0,
               None) == lnf4.LNF4_EINVAL  # dy missing


def test_group_validation(L):
    p = lnf4.make_proj(_weight(), y=FAKE)
    q = lnf4.make_proj(_weight(in_f=256), y=FAKE)
    arr = (lnf4.lnf4_proj * 2)(p, q)
    assert L.lora_group_fwd(arr, 2, FAKE, 4, 1, None) == lnf4.LNF4_ESHAPE   # different in_f
    assert L.lora_group_fwd(arr, 9, FAKE, 4, 1, None) == lnf4.LNF4_EINVAL
    assert L.lora_group_fwd(arr, 0, FAKE, 4, 1, None) == lnf4.LNF4_EINVAL
    one = (lnf4.lnf4_proj * 1)(p)
    for bad in (-1, 3):   # adapters_enabled: 0 off, 1 on, 2 on with u given
        assert L.lora_group_fwd(one, 1, FAKE, 4, bad, None) == lnf4.LNF4_EINVAL


def test_shard_layout():
    outs = [896, 128, 128, 896, 4864, 4864, 896]
    ins = [896, 896, 896, 896, 896, 896, 4864]
    offs, total = lnf4.lnf4_shard_layout(outs, ins, lnf4.FMT_NF4)
    assert all(o % 256 == 0 for o in offs)
    P = sum(o * i for o, i in zip(outs, ins))
    assert P == 14_909_440
    # codes (P/2) + absmax (P/64 * 4), each section padded to 256 bytes
    assert P // 2 + P // 16 <= total <= P // 2 + P // 16 + 256 * 14
    for p in range(7):
        n = outs[p] * ins[p]
        assert offs[2 * p + 1] - offs[2 * p] >= n // 2
    offs, total = lnf4.lnf4_shard_layout(outs, ins, lnf4.FMT_BF16)
    assert offs[1] == -1 and total >= 2 * P
    with pytest.raises(lnf4.LNF4Error):
        lnf4.lnf4_shard_layout([16], [100], lnf4.FMT_NF4)


def test_stream_validation(L):
    out = ctypes.c_void_p()
    hs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    sb = (ctypes.c_size_t * 2)(1024, 1024)
    db = (ctypes.c_void_p * 9)(*([FAKE] * 9))
    sc = (ctypes.c_int32 * 4)(0, 1, 1, 0)
    args = lambda nb, sched=sc, sl=4, bb=4096, res=0: L.stream_create(hs, sb, 2, db, bb, nb, sched, sl, res, None,
                                                                      None, 0, ctypes.byref(out))
    assert args(9) == lnf4.LNF4_EINVAL           # more than 8 buffers
    assert args(1) == lnf4.LNF4_EINVAL           # fewer than 2
    assert args(2, bb=512) == lnf4.LNF4_ESHAPE   # shard larger than a buffer
    bad = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert args(2, sched=bad) == lnf4.LNF4_EINVAL  # schedule names a missing shard
    assert args(3, res=1) == lnf4.LNF4_EINVAL    # resident needs one buffer per shard
    assert args(2, res=3) == lnf4.LNF4_EINVAL    # mode outside ring / resident / reuse
    assert args(2, res=-1) == lnf4.LNF4_EINVAL
    assert args(9, res=2) == lnf4.LNF4_EINVAL    # reuse keeps the 2..8 buffer range
    db2 = (ctypes.c_void_p * 2)(FAKE + 16, FAKE)
    assert L.stream_create(hs, sb, 2, db2, 4096, 2, sc, 4, 0, None, None, 0, ctypes.byref(out)) == lnf4.LNF4_EALIGN
    p = ctypes.c_void_p()
    assert L.stream_layer_step(None, 0, None, ctypes.byref(p)) == lnf4.LNF4_ESTATE
    assert L.stream_slot_load_part(None, 0, 0, 4, None) == lnf4.LNF4_ESTATE
    assert L.stream_slot_load(None, 0, None) == lnf4.LNF4_ESTATE
    assert L.stream_slot_wait(None, None, ctypes.byref(p)) == lnf4.LNF4_ESTATE
    assert L.stream_destroy(None) == lnf4.LNF4_OK


def test_stream_disk_validation(L, tmp_path):
    # the disk tier rejects bad arguments before any HIP call (the file is opened and
    # sized first; page-locking is checked last)
    f = tmp_path / "shards.bin"
    f.write_bytes(bytes(3 * 4096))
    out = ctypes.c_void_p()
    sb = (ctypes.c_size_t * 2)(4096, 4096)
    db = (ctypes.c_void_p * 2)(FAKE, FAKE)
    sc = (ctypes.c_int32 * 4)(0, 1, 1, 0)
    stg = (ctypes.c_void_p * 9)(*([FAKE] * 9))

    def call(path=str(f), offs=(0, 4096), n_stage=2, stage_bytes=4096, sched=sc, stages=stg):
        fo = (ctypes.c_int64 * 2)(*offs)
        return L.stream_create_disk(path.encode(), fo, 1, stages, stage_bytes, n_stage, None, sb, 2, db, 4096,
                                    2, sched, 4, None, None, 0, ctypes.byref(out))

    assert call(n_stage=0) == lnf4.LNF4_EINVAL                   # read-ahead depth 1..8
    assert call(n_stage=9) == lnf4.LNF4_EINVAL
    assert call(stage_bytes=2048) == lnf4.LNF4_ESHAPE            # a shard larger than staging
    assert call(path=str(tmp_path / "missing.bin")) == lnf4.LNF4_EINVAL
    assert call(offs=(0, 3 * 4096)) == lnf4.LNF4_ESHAPE          # shard 1 ends past the file
    assert call(offs=(0, -4096)) == lnf4.LNF4_EINVAL
    assert call(stages=(ctypes.c_void_p * 2)(FAKE, None)) == lnf4.LNF4_EINVAL  # a NULL staging buffer
    bad = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert call(sched=bad) == lnf4.LNF4_EINVAL                   # schedule names a missing shard
    b, t = ctypes.c_int64(), ctypes.c_double()
    assert L.stream_disk_stats(None, ctypes.byref(b), ctypes.byref(t)) == lnf4.LNF4_ESTATE


def test_size_limits(L):
    # a weight or activation beyond 2^31-1 bytes is rejected before any HIP call
    big = lnf4.make_weight(lnf4.FMT_BF16, FAKE, None, 1 << 16, 1 << 15, 64)  # 2^32 bytes of bf16
    assert L.lora_linear_fwd(ctypes.byref(big), FAKE, 16, None, None, 0, 0.0, FAKE, None, None) == lnf4.LNF4_ESHAPE
    w = lnf4.make_weight(lnf4.FMT_NF4, FAKE, FAKE, 1024, 1 << 20, 64)       # codes 2^29 bytes: fine
    assert L.lora_linear_fwd(ctypes.byref(w), FAKE, 1 << 11, None, None, 0, 0.0, FAKE, None, None) \
        == lnf4.LNF4_ESHAPE                                                 # x: 2^11 x 2^20 bf16 = 2^32 bytes


def test_output_side_validation(L):
    # embedding gather
    assert L.lnf4_embed_gather(FAKE, 100, 12, FAKE, 4, FAKE, None) == lnf4.LNF4_ESHAPE    # hidden % 8
    assert L.lnf4_embed_gather(FAKE, 0, 16, FAKE, 4, FAKE, None) == lnf4.LNF4_ESHAPE      # empty vocab
    assert L.lnf4_embed_gather(None, 100, 16, FAKE, 4, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_embed_gather(FAKE + 2, 100, 16, FAKE, 4, FAKE, None) == lnf4.LNF4_EALIGN
    assert L.lnf4_embed_gather(FAKE, 100, 16, FAKE, -1, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_embed_gather(None, 100, 16, None, 0, None, None) == lnf4.LNF4_OK        # T = 0: no-op
    # cross-entropy
    ce = L.lnf4_cross_entropy
    assert ce(FAKE, 4, 100, FAKE, 1.0, None, 1, FAKE, FAKE, None) == lnf4.LNF4_ESHAPE     # V % 8
    assert ce(FAKE, 4, 96, FAKE, 1.0, None, 1, None, None, None) == lnf4.LNF4_EINVAL      # nothing asked for
    assert ce(FAKE, 4, 96, None, 1.0, None, 1, FAKE, None, None) == lnf4.LNF4_EINVAL      # labels missing
    assert ce(FAKE, 4, 96, FAKE, 1.0, FAKE, 0, FAKE, None, None) == lnf4.LNF4_EINVAL      # rows_per_scale
    assert ce(FAKE, 4, 96, FAKE, float("nan"), None, 1, FAKE, None, None) == lnf4.LNF4_EINVAL
    assert ce(FAKE + 8, 4, 96, FAKE, 1.0, None, 1, FAKE, None, None) == lnf4.LNF4_EALIGN
    assert ce(FAKE, 4, 96, FAKE, 1.0, None, 1, None, FAKE + 2, None) == lnf4.LNF4_EALIGN
    assert ce(None, 0, 96, None, 1.0, None, 1, None, None, None) == lnf4.LNF4_OK
    # sequence sums and the preference loss
    assert L.lnf4_sequence_sums(FAKE, 2, 0, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_sequence_sums(FAKE, -1, 8, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_sequence_sums(None, 0, 8, None, None) == lnf4.LNF4_OK
    assert L.lnf4_dpo_loss(FAKE, FAKE, 0, 0.1, FAKE, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_dpo_loss(FAKE, FAKE, 2, 0.0, FAKE, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_dpo_loss(FAKE, None, 2, 0.1, FAKE, FAKE, None) == lnf4.LNF4_EINVAL
    assert L.lnf4_dpo_loss(FAKE, FAKE, 2, 0.1, FAKE + 1, FAKE, None) == lnf4.LNF4_EALIGN


def test_decoder_glue_validation(L):
    E = lnf4
    assert L.lnf4_rmsnorm_fwd(FAKE, 4, 12, FAKE, 1e-5, FAKE, FAKE, None) == E.LNF4_ESHAPE      # H % 8
    assert L.lnf4_rmsnorm_fwd(FAKE, 4, 16, FAKE, -1.0, FAKE, FAKE, None) == E.LNF4_EINVAL      # eps
    assert L.lnf4_rmsnorm_fwd(FAKE + 8, 4, 16, FAKE, 1e-5, FAKE, None, None) == E.LNF4_EALIGN
    assert L.lnf4_rmsnorm_fwd(None, 0, 16, None, 1e-5, None, None, None) == E.LNF4_OK          # T = 0
    assert L.lnf4_rmsnorm_bwd(FAKE, 4, 16, FAKE, None, FAKE, None, FAKE, None) == E.LNF4_EINVAL  # rstd
    assert L.lnf4_rope_table(64, 24, 1e4, FAKE, None) == E.LNF4_ESHAPE                         # D % 16
    assert L.lnf4_rope_table(64, 64, 1.0, FAKE, None) == E.LNF4_EINVAL                         # base
    assert L.lnf4_rope(FAKE, 4, 2, 64, 0, FAKE, 0, None) == E.LNF4_EINVAL                      # seq_len
    assert L.lnf4_swiglu_fwd(FAKE, FAKE, 12, FAKE, None) == E.LNF4_ESHAPE
    assert L.lnf4_swiglu_bwd(FAKE, FAKE, None, 16, FAKE, FAKE, None) == E.LNF4_EINVAL
    assert L.lnf4_add(FAKE, FAKE + 4, 16, FAKE, None) == E.LNF4_EALIGN
    fwd = L.lnf4_attn_fwd
    assert fwd(FAKE, FAKE, FAKE, 128, 4, 2, 96, 64, FAKE, FAKE, None) == E.LNF4_ESHAPE   # head_dim
    assert fwd(FAKE, FAKE, FAKE, 128, 6, 4, 64, 64, FAKE, FAKE, None) == E.LNF4_ESHAPE   # heads not grouped
    assert fwd(FAKE, FAKE, FAKE, 128, 4, 2, 64, 48, FAKE, FAKE, None) == E.LNF4_ESHAPE   # seq_len % 64
    assert fwd(FAKE, FAKE, FAKE, 160, 4, 2, 64, 64, FAKE, FAKE, None) == E.LNF4_ESHAPE   # T % seq_len
    assert fwd(FAKE, FAKE, FAKE, 128, 4, 2, 64, 64, FAKE, None, None) == E.LNF4_EINVAL
    assert L.lnf4_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 4, 2, 64, 64, FAKE, FAKE, FAKE, None, 0,
                           None) == E.LNF4_EINVAL                                         # workspace
    need = L.lnf4_attn_bwd_workspace(128, 4, 2, 64)
    assert need == 4 * 128 * 4 + 2 * 4 * 128 * 64 * 4                                     # rowsums + fp32 shares
    assert L.lnf4_attn_bwd_workspace(128, 4, 4, 64) == 4 * 128 * 4                        # no grouping: no shares
    assert L.lnf4_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 4, 2, 64, 64, FAKE, FAKE, FAKE, FAKE, need - 1,
                           None) == E.LNF4_ESHAPE


def test_group_fwd_workspace_and_validation(L):
    """The K-split forward's workspace query (host-only; a host with no GPU counts 256
    compute units) and its workspace checks, which come before any launch."""
    def projs(fmt, out_f, in_f, n=1):
        return [lnf4.make_proj(_weight(fmt=fmt, out_f=out_f, in_f=in_f), y=FAKE) for _ in range(n)]

    # the SwiGLU down projection of a Qwen2.5-0.5B layer at T = 2048: 16 x 4 tiles of 128 x 256
    # over 76 K-blocks run as 4 splits, one fp32 [T, 896] array of sums per split
    assert lnf4.lora_group_fwd_workspace(projs(0, 896, 4864), 2048) == 4 * 2048 * 896 * 4
    assert lnf4.lora_group_fwd_workspace(projs(1, 896, 4864), 2048) == 0        # bf16 weights
    # the Llama-8B down projection: 8 x 16 tiles of 256 x 256 over 224 K-blocks run as 2 splits
    assert lnf4.lora_group_fwd_workspace(projs(0, 4096, 14336), 2048) == 2 * 2048 * 4096 * 4
    assert lnf4.lora_group_fwd_workspace(projs(0, 4096, 4096), 2048) == 0       # 64 K-blocks: too short
    assert lnf4.lora_group_fwd_workspace(projs(0, 4300, 8192), 1000) == 2 * 1000 * 4300 * 4  # 256-row, 2 splits
    assert lnf4.lora_group_fwd_workspace(projs(0, 28672, 4096), 2048) == 0      # 896 tiles: not split
    # two projections, 4 x 18 tiles of 256 rows over 256 K-blocks: 3 splits (3 x 72 tiles)
    assert lnf4.lora_group_fwd_workspace(projs(0, 2200, 16384) + projs(0, 2100, 16384), 1000) == \
        3 * 1000 * (2200 + 2100) * 4
    assert lnf4.lora_group_fwd_workspace(projs(0, 896, 896), 2048) == 0         # 14 K-blocks: too short
    assert lnf4.lora_group_fwd_workspace(projs(0, 904, 2112, 2), 200) == 4 * 200 * 904 * 4 * 2
    assert lnf4.lora_group_fwd_workspace(projs(0, 896, 4864), 0) == 0
    need = lnf4.lora_group_fwd_workspace(projs(0, 896, 4864), 2048)
    arr, n = lnf4._proj_array(projs(0, 896, 4864))
    ws = L.lora_group_fwd_ws
    assert ws(arr, n, FAKE, 2048, 1, None, need, None) == lnf4.LNF4_EINVAL
    assert ws(arr, n, FAKE, 2048, 1, FAKE, need - 1, None) == lnf4.LNF4_ESHAPE
    assert ws(arr, n, FAKE, 2048, 1, FAKE + 16, need, None) == lnf4.LNF4_EALIGN
