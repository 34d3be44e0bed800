"""GPU parity of the work split (pa_set_work_split): phase-1 items cut into pieces
whose partial states phase 2 folds.  Same bar as the other parity tests; a piece's
partial state is checked against the float64 oracle's partials at partition size
P / pieces, which is exactly the token range the piece covers."""
import sys

import numpy as np
import pytest

import oracle
import split_rule
from paged_split_kv_pa_amd import binding as B
from paged_split_kv_pa_amd import workloads as wl

from helpers import check_close, small_workload, to_f64, upload, work_split

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def decode_v2(w, dev, P, max_context_len=0, ws=None):
    if ws is None:
        lay = B.workspace_layout(dev["q"], dev["k_cache"], dev["block_tables"],
                                 max_context_len, P)
        ws = torch.zeros(lay["bytes"], dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    B.pa_decode_ex(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                   dev["context_lens"], w.scale, P, workspace=ws,
                   max_context_len=max_context_len, path=B.PA_PATH_V2)
    torch.cuda.synchronize()
    return out, ws


def reference(w):
    return oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                   w.scale, w.dtype)


_CFG = {}


def config_case(i):
    if i not in _CFG:
        w = wl.config(i)
        _CFG[i] = (w, upload(w), reference(w))
    return _CFG[i]


FORCED = [(c, k, f) for c in (0, 1, 4) for k in (2, 8) for f in ("all", "mid")]


@pytest.mark.parametrize("cfg,pieces,first", FORCED,
                         ids=[f"{wl.CONFIG_NAMES[c]}-k{k}-{f}" for c, k, f in FORCED])
def test_forced_split_matches_oracle(cfg, pieces, first):
    w, dev, ref = config_case(cfg)
    P = 512
    items = w.num_seqs * w.num_kv_heads * -(-w.max_blocks_per_seq * 16 // P)
    f0 = 0 if first == "all" else items // 2 + 1
    with work_split(pieces, f0):
        plan = B.split_plan(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
        say(f"forced split {wl.CONFIG_NAMES[cfg]} pieces={pieces} first={f0} plan={plan}")
        assert (plan["first"], plan["pieces"], plan["workgroups"]) == \
            split_rule.plan(items, P, pieces, f0)
        out, _ = decode_v2(w, dev, P)
    check_close(to_f64(out), ref, f"split {wl.CONFIG_NAMES[cfg]} k={pieces} first={f0}")


SPLIT_EDGE = [("f32", 128, 1), ("f32", 256, 2), ("f16", 128, 16), ("bf16", 256, 8),
              ("bf16", 128, 4)]


@pytest.mark.parametrize("dtype,D,G", SPLIT_EDGE, ids=[f"{a}-d{b}-g{c}" for a, b, c in SPLIT_EDGE])
def test_split_edge_contexts(dtype, D, G):
    ctx = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000]
    w = small_workload(300 + G + D, ctx, Hq=2 * G, Hkv=2, D=D, dtype=dtype)
    dev = upload(w)
    ref = reference(w)
    for P, pieces, f0 in ((128, 2, 0), (512, 8, 0), (512, 4, 7), (256, 4, 19), (1024, 16, 3)):
        with work_split(pieces, f0):
            say(f"split edge dtype={dtype} D={D} G={G} P={P} pieces={pieces} first={f0}")
            got = to_f64(decode_v2(w, dev, P)[0])
        check_close(got, ref, f"split edge {dtype} D={D} G={G} P={P} k={pieces}")
        assert np.all(got[0] == 0), "empty sequence must give 0"


@pytest.mark.parametrize("dtype,G,pieces,P", [("bf16", 8, 4, 512), ("f32", 1, 16, 1024),
                                              ("f16", 4, 2, 512), ("bf16", 16, 8, 512)])
def test_piece_partials_match_oracle_subpartitions(dtype, G, pieces, P):
    """Every non-empty piece slot holds the oracle's partial of its token range."""
    ctx = [1000, 333, 16, 1, 0, 700]
    Hkv = 2
    w = small_workload(77 + G, ctx, Hq=Hkv * G, Hkv=Hkv, D=128, dtype=dtype)
    dev = upload(w)
    with work_split(pieces, 0):
        plan = B.split_plan(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
        say(f"piece partials dtype={dtype} G={G} pieces={pieces} plan={plan}")
        assert plan["first"] == 0 and plan["pieces"] == pieces
        out, ws = decode_v2(w, dev, P)
    lay = B.workspace_layout(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
    raw = ws.cpu().numpy()

    def view(name):
        off, shape = lay[name]
        n = int(np.prod(shape))
        return raw[off:off + 4 * n].view(np.float32).reshape(shape).astype(np.float64)

    po, pm, ps = view("piece_out"), view("piece_max"), view("piece_sum")
    sub = P // pieces
    _, parts = oracle.partitioned_decode(w.q, w.k_cache, w.v_cache, w.block_tables,
                                         w.context_lens, w.scale, w.dtype, sub)
    pmax = lay["pmax"]
    checked = 0
    for b, n in enumerate(ctx):
        for h in range(Hkv):
            for p in range(pmax):
                for c in range(pieces):
                    r = p * pieces + c  # sub-partition index of this piece
                    if r * sub >= n:
                        continue  # empty piece: its slot is never written nor read
                    slot = (p + pmax * (h + Hkv * b)) * pieces + c
                    for gq in range(G):
                        hq = h * G + gq
                        np.testing.assert_allclose(pm[slot, gq], parts["max_logits"][b, hq, r],
                                                   rtol=1e-5, atol=1e-4)
                        np.testing.assert_allclose(ps[slot, gq], parts["exp_sums"][b, hq, r],
                                                   rtol=2e-4)
                        check_close(po[slot, gq][None, None], parts["tmp_out"][b, hq, r][None, None],
                                    f"piece b={b} h={h} p={p} c={c} g={gq}")
                        checked += 1
    assert checked > 0
    check_close(to_f64(out), reference(w), "piece-partials output")


def test_automatic_split_of_the_tail_items():
    """272 items on 256 compute units: the last 16 are cut, starting inside a row."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    w = small_workload(91, [8200, 8000], Hq=64, Hkv=8, D=128, dtype="bf16")
    dev = upload(w)
    P = 512
    pmax = -(-w.max_blocks_per_seq * 16 // P)
    items = 2 * 8 * pmax
    with work_split(-1):
        plan = B.split_plan(dev["q"], dev["k_cache"], dev["block_tables"], 0, P)
        say(f"automatic split ncu={ncu} items={items} plan={plan}")
        assert (plan["first"], plan["pieces"], plan["workgroups"]) == \
            split_rule.plan(items, P, -1, ncu=ncu)
        if ncu == 256:
            assert items == 272 and plan["first"] == 256 and plan["pieces"] == 8
        got, _ = decode_v2(w, dev, P)
        again, _ = decode_v2(w, dev, P)
    with work_split(0):
        whole, _ = decode_v2(w, dev, P)
    ref = reference(w)
    check_close(to_f64(got), ref, "automatic split")
    check_close(to_f64(whole), ref, "no split")
    assert torch.equal(got, again), "split runs must be bitwise deterministic"


@pytest.mark.parametrize("cfg", [2, 1])
def test_automatic_split_on_workloads(cfg):
    """long_100k (784 items: the last 16 cut) and single_8k (64 items: all cut)."""
    w, dev, ref = config_case(cfg)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    with work_split(-1):
        plan = B.split_plan(dev["q"], dev["k_cache"], dev["block_tables"], 0, 512)
        say(f"automatic split {wl.CONFIG_NAMES[cfg]} ncu={ncu} plan={plan}")
        assert (plan["first"], plan["pieces"], plan["workgroups"]) == \
            split_rule.plan(plan["items"], 512, -1, ncu=ncu)
        got, _ = decode_v2(w, dev, 512)
    with work_split(0):
        whole, _ = decode_v2(w, dev, 512)
    check_close(to_f64(got), ref, f"split {wl.CONFIG_NAMES[cfg]}")
    check_close(to_f64(got), to_f64(whole), f"split vs whole {wl.CONFIG_NAMES[cfg]}")


@pytest.mark.parametrize("pieces", [0, 2])
def test_context_beyond_the_hint_attends_a_prefix(pieces):
    """Contexts longer than max_context_len: V2 attends the first ceil(hint/P)*P tokens,
    V1 the first hint rounded up to 16 (the header's contract), with or without a cut."""
    ctx = [1000, 333, 40]
    w = small_workload(123, ctx, Hq=16, Hkv=2, D=128, dtype="bf16")
    dev = upload(w)
    hint, P = 300, 128
    with work_split(pieces, 0):
        say(f"context beyond hint pieces={pieces}")
        v2, _ = decode_v2(w, dev, P, max_context_len=hint)
        v1 = torch.empty_like(dev["q"])
        B.pa_decode_ex(v1, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                       dev["context_lens"], w.scale, P, max_context_len=hint,
                       path=B.PA_PATH_V1)
        torch.cuda.synchronize()
    for got, keep in ((v2, -(-hint // P) * P), (v1, -(-hint // 16) * 16)):
        lens = np.minimum(np.array(ctx), keep).astype(np.int32)
        ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_tables, lens, w.scale,
                                      w.dtype)
        check_close(to_f64(got), ref, f"prefix of {keep} tokens, pieces={pieces}")
