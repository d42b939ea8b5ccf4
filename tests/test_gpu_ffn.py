"""GPU parity of moe_mxfp4_ffn (and route -> FFN end to end) against the fp64 oracle.

Bar (per token set): relative L2 error <= 2e-3 and max abs error <= 1e-2 * max|ref|.
Small configs are compared on every output; the K3-shaped configs (896
experts resident, the launch configuration the benchmark times) on sampled
tokens, which the oracle evaluates one expert at a time.
"""

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs.device import upload_experts
from oracle.ffn import ffn_ref
from oracle.route import route_ref
from tests.gpu_util import assert_ffn_close, bf16_dev, expert_blocks, to_dev_u8

pytestmark = pytest.mark.gpu


class HostExperts:
    """Source-layout experts held in host memory (small configs)."""

    def __init__(self, cfg):
        self.src = moe_inputs.ExpertSource(cfg)
        self.mats = [self.src[e] for e in range(cfg.E)]

    def __getitem__(self, e):
        return self.mats[e]

    def __len__(self):
        return len(self.mats)


def device_experts(k3, cfg):
    return upload_experts(cfg, expert_blocks(k3))


def run_ffn(k3, dev, x_bits, ids, w):
    out = k3.moe_mxfp4_ffn(bf16_dev(x_bits), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                           dev.w1, dev.w3, dev.w2)
    return out.cpu().numpy()


def small_case(k3, cfg, ids=None, w=None):
    batch = moe_inputs.make_batch(cfg)
    if ids is None:
        ids, w = route_ref(batch.z, batch.b, cfg.k)
    dev = device_experts(k3, cfg)
    got = run_ffn(k3, dev, batch.x, ids.astype(np.int32), w.astype(np.float32))
    ref = ffn_ref(batch.x, ids, w, HostExperts(cfg))
    return got, ref, batch, dev


def test_tiny(k3):
    print("[ffn] tiny", flush=True)
    got, ref, _, _ = small_case(k3, moe_inputs.TINY)
    assert_ffn_close(got, ref, "tiny")


@pytest.mark.parametrize(
    "E,k,D,I,T",
    [
        (16, 4, 512, 384, 200),  # 64-row tiles with ragged tails, 4 D-segments, partial last segment
        (8, 2, 128, 256, 100),  # 32-row tiles
        (5, 1, 256, 128, 1),  # single token, k = 1
        (12, 3, 640, 512, 65),  # two grouping chunks, one token in the second
        (8192, 2, 128, 128, 40),  # largest supported expert count
        (8, 2, 512, 512, 300),  # large-tile path: ragged 128-row (gate/up) and 64-row (down) tiles
        (16, 4, 1024, 512, 400),  # large-tile path with two feature tiles per matrix
        (12, 4, 2048, 1024, 700),  # large-tile path, 4 gate/up feature tiles (2D work order)
        (12, 8, 1024, 512, 2100),  # 16800 entries: 128-row down tiles, ragged last tiles
        (64, 4, 512, 512, 8),  # weight-streaming path: about one row per expert
        (16, 4, 1024, 512, 16),  # streaming path: ~4 rows per expert, experts split over 4-row tiles
        (32, 8, 1536, 1024, 3),  # streaming path: 3 K stages (gate/up), 2 (down)
        (896, 16, 512, 1024, 1),  # streaming path: one token, 16 experts of 896
        (4, 2, 512, 512, 8),  # streaming-only batch: experts of up to 8 rows over several 4- and 2-row tiles
        (3, 3, 512, 1024, 5),  # streaming-only batch: every expert has all 5 rows
        (4, 2, 512, 512, 9),  # one token past the streaming-only batch: large-tile kernels for experts of 5+ rows
        (200, 64, 512, 512, 4),  # grouping inside the gate/up launch: 256 entries, one per thread
        (200, 64, 512, 512, 8),  # grouping inside the gate/up launch at its limit: 512 entries
        (8, 2, 96, 160, 50),  # D, I multiples of 32 only: odd block counts (unaligned rows), a 32-feature tile
        (6, 3, 224, 288, 70),  # 7 and 9 blocks per row, 224 / 288 outputs (a partial last feature tile)
        (4, 2, 32, 32, 10),  # one block per row, one 32-feature tile
        (8, 2, 384, 640, 33),  # 12 and 20 blocks per row (4-byte rows, a partial last K segment)
        (5, 2, 544, 96, 130),  # 17 blocks per row: one full K segment plus one block
    ],
)
def test_shapes(k3, E, k, D, I, T):
    print(f"[ffn] shape E={E} k={k} D={D} I={I} T={T}", flush=True)
    cfg = moe_inputs.TINY.with_(E=E, k=k, D=D, I=I, T=T, config_id=40)
    got, ref, _, _ = small_case(k3, cfg)
    assert_ffn_close(got, ref, f"E={E} k={k} D={D} I={I} T={T}")


def test_hot_expert_invalid_and_duplicate_ids(k3):
    cfg = moe_inputs.TINY.with_(E=6, k=3, T=300, config_id=41)
    g = np.random.default_rng(11)
    ids = g.integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)
    ids[:, 0] = 2  # one hot expert: every token, 5 tiles of 64 rows
    ids[::7, 1] = -1  # out of range -> skipped
    ids[::5, 2] = cfg.E + 4
    ids[1::3, 2] = ids[1::3, 0]  # repeats an earlier slot -> skipped
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    got, ref, batch, dev = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "hot/invalid/duplicate")
    # all entries invalid -> exact zeros
    bad = np.full_like(ids, -5)
    out = run_ffn(k3, dev, batch.x, bad, w)
    assert np.all(out == 0)
    # determinism: bitwise-identical reruns
    a = run_ffn(k3, dev, batch.x, ids, w)
    b = run_ffn(k3, dev, batch.x, ids, w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("T", [8, 4])  # grouped in the gate/up launch: x re-laid out first / x read in place
def test_streaming_path_hot_invalid_and_duplicate_ids(k3, T):
    # decode-sized batch (at most 4 rows per active expert on average) with one
    # expert in every row: its T rows span one or two 4-row tiles
    print(f"[ffn] streaming hot/invalid/duplicate T={T}", flush=True)
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=512, T=T, config_id=42)
    g = np.random.default_rng(13)
    ids = np.stack([g.permutation(cfg.E)[: cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    ids[:, 0] = 5
    rest = ids[:, 1:]  # a view: keep the hot expert in slot 0 only
    rest[rest == 5] = 6
    ids[3, 1] = -2  # out of range -> skipped
    ids[2, 3] = ids[2, 2]  # repeat -> skipped
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    got, ref, batch, dev = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "streaming hot/invalid/duplicate")
    a = run_ffn(k3, dev, batch.x, ids, w)
    assert np.array_equal(a.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("T,D,I", [(3, 512, 512), (8, 512, 512), (40, 128, 256)])
def test_nan_and_inf_weights_on_skipped_entries(k3, T, D, I):
    # an entry that is skipped (id out of range, or a repeat within its row)
    # contributes nothing whatever its weight: NaN and inf there must not
    # reach the output (streaming path grouped in the gate/up launch with x
    # read in place / re-laid out, and the small-tile path)
    print(f"[ffn] NaN/inf weights on skipped entries T={T} D={D} I={I}", flush=True)
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=D, I=I, T=T, config_id=49)
    g = np.random.default_rng(19)
    ids = np.stack([g.permutation(cfg.E)[: cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    ids[0, 1] = -1
    w[0, 1] = np.nan
    ids[1, 3] = cfg.E + 2
    w[1, 3] = np.inf
    ids[2, 2] = ids[2, 0]  # repeat -> skipped
    w[2, 2] = np.nan
    ids[T - 1, 3] = ids[T - 1, 1]
    w[T - 1, 3] = -np.inf
    got, ref, _, _ = small_case(k3, cfg, ids, w)
    assert np.all(np.isfinite(ref))
    assert_ffn_close(got, ref, f"NaN/inf on skipped entries T={T} D={D}")


def test_self_grouping_duplicates_and_invalid_ids(k3):
    # 3 tokens x 8 slots drawn from 6 experts with repeats (the grouping inside
    # the gate/up launch skips repeats of a row), plus ids outside [0, E)
    print("[ffn] self-grouping with repeated and invalid ids", flush=True)
    cfg = moe_inputs.TINY.with_(E=40, k=8, D=512, I=512, T=3, config_id=47)
    g = np.random.default_rng(17)
    ids = g.integers(0, 6, size=(cfg.T, cfg.k)).astype(np.int32)
    ids[0, 5] = cfg.E  # out of range
    ids[2, 0] = -1
    ids[1, :] = 4  # one expert, every slot: a single valid entry
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    got, ref, batch, dev = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "self-grouping repeats/invalid")
    again = run_ffn(k3, dev, batch.x, ids, w)
    assert np.array_equal(again.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("T", [1, 3, 8])
def test_decode_outputs_whatever_the_workspace_holds(k3, T):
    # decode batches (grouped inside the gate/up launch): the workspace starts
    # as 0xFF bytes and the output as NaN, so state the launches failed to set
    # or an output the combine failed to write shows; a second call reuses the
    # workspace.  A token whose every slot is skipped gets zeros, and a batch
    # of only skipped entries (no tiles at all) all zeros.
    print(f"[ffn] decode outputs over a dirty workspace T={T}", flush=True)
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=1024, T=T, config_id=50)
    g = np.random.default_rng(23)
    ids = np.stack([g.permutation(cfg.E)[: cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    if T > 1:
        ids[T // 2, :] = -1  # every slot skipped
    batch = moe_inputs.make_batch(cfg)
    dev = device_experts(k3, cfg)
    ref = ffn_ref(batch.x, ids, w, HostExperts(cfg))
    x = bf16_dev(batch.x)
    need = k3.moe_mxfp4_ffn_workspace_size(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        out = torch.full((cfg.T, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        k3.moe_mxfp4_ffn(x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), dev.w1, dev.w3, dev.w2,
                         out=out, workspace=ws)
        outs.append(out.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert_ffn_close(outs[0], ref, f"decode over a dirty workspace T={T}")
    if T > 1:
        assert np.all(outs[0][T // 2] == 0)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    bad = np.full_like(ids, cfg.E + 1)
    out = torch.full((cfg.T, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
    k3.moe_mxfp4_ffn(x, torch.from_numpy(bad).cuda(), torch.from_numpy(w).cuda(), dev.w1, dev.w3, dev.w2,
                     out=out, workspace=ws)
    assert np.all(out.cpu().numpy() == 0)


def test_mixed_large_and_streaming_experts(k3):
    # one call in which some experts have many rows (large-tile kernels, with a
    # partial last token group) and others a few rows (weight-streaming kernels)
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=1024, T=90, config_id=44)
    g = np.random.default_rng(14)
    ids = np.stack([g.permutation(cfg.E)[: cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    ids[:, 0] = 3  # 90 rows: one full 64-row down tile + a partial one, 1 gate/up tile of 90
    ids[:37, 1] = 7  # 37 rows
    rest = ids[:, 2:]
    rest[(rest == 3) | (rest == 7)] = 11
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    got, ref, _, _ = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "mixed large/streaming")


def test_shared_streaming_tiles_around_their_limits(k3):
    # grouped batch (more than 8 tokens): experts of at most 16 rows go to the
    # shared-tile streaming kernels (16-row gate/up, 8-row down tiles), larger
    # ones to the large-tile kernels.  Row counts 1, 4, 8, 9, 15, 16 (one
    # gate/up tile; one or two down tiles, ragged), 17 (just past the limit)
    # and 40; every token checked
    cfg = moe_inputs.TINY.with_(E=24, k=4, D=512, I=1024, T=64, config_id=49)
    g = np.random.default_rng(16)
    ids = np.full((cfg.T, cfg.k), -1, np.int32)
    col = {}
    t0 = 0
    for e, n in ((0, 1), (1, 4), (2, 8), (3, 9), (4, 15), (5, 16), (6, 17), (7, 40)):
        rows = (t0 + np.arange(n)) % cfg.T
        t0 += n
        for t in rows:
            j = col.get(t, 0)
            ids[t, j] = e
            col[t] = j + 1
    # the free slots go to experts 8..23 (9 or 10 rows each), no repeats in a row
    free = np.argwhere(ids < 0)
    fill = 8 + np.arange(len(free)) % 16
    for (t, j), e in zip(free, fill):
        ids[t, j] = e if e not in ids[t] else -1
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    counts = [int((ids == e).sum()) for e in range(8)]
    assert counts == [1, 4, 8, 9, 15, 16, 17, 40], counts
    print(f"[ffn] shared streaming tiles around their limits", flush=True)
    got, ref, _, _ = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "shared streaming tiles")


def test_large_batch_mixed_with_few_row_experts(k3):
    # 16384 routed entries (128-row large-tile down tiles) with experts of
    # 1..5 rows (weight-streaming kernels) in the same call
    cfg = moe_inputs.TINY.with_(E=40, k=8, D=512, I=512, T=2048, config_id=45)
    g = np.random.default_rng(15)
    ids = np.stack([g.permutation(30)[: cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    ids[0, 7] = 30  # 1 row
    ids[1:3, 7] = 31  # 2 rows
    ids[3:6, 7] = 32  # 3 rows
    ids[6:10, 7] = 33  # 4 rows
    ids[10:15, 7] = 34  # 5 rows
    ids[2000, 7] = 39  # 1 row, in the last token group
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    print(f"[ffn] large batch with few-row experts T={cfg.T}", flush=True)
    got, ref, _, _ = small_case(k3, cfg, ids, w)
    assert_ffn_close(got, ref, "large batch, few-row experts")


def test_side_stream_matches_serial_launches(k3):
    # 24 large-tile + 12 streaming experts: moe_mxfp4_ffn runs the streaming
    # launches on a side stream; the profiled entry point runs every launch on
    # the caller's stream.  Both must give the same bits.
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=512, T=90, config_id=43)
    print("[ffn] side stream vs serial launches", flush=True)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    dev = device_experts(k3, cfg)
    x = bf16_dev(batch.x)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w.astype(np.float32)).cuda()
    conc = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(k3.FFN_STAGE_EVENTS)]
    serial = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2, stage_events=events)
    torch.cuda.synchronize()
    assert torch.equal(conc.view(torch.int32), serial.view(torch.int32))
    for _ in range(3):  # repeated concurrent calls stay bit-identical
        again = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), conc.view(torch.int32))


def _mixed_inputs(k3):
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=512, T=90, config_id=43)  # 24 large-tile + 12 streaming
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    dev = device_experts(k3, cfg)
    x = bf16_dev(batch.x)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w.astype(np.float32)).cuda()
    return cfg, dev, x, ids_d, w_d


def test_side_streams_of_concurrent_threads(k3):
    # two host threads, each on its own stream with its own buffers (and its
    # own side stream): the same bits as one call on the main thread
    import threading
    cfg, dev, x, ids_d, w_d = _mixed_inputs(k3)
    ref = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                outs = [k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2) for _ in range(4)]
            st.synchronize()
            results[i] = [o.cpu() for o in outs]
        except Exception as exc:  # surfaced below
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    want = ref.cpu().view(torch.int32)
    for i in range(2):
        for o in results[i]:
            assert torch.equal(o.view(torch.int32), want)


def test_first_call_of_a_thread_inside_capture(k3):
    # a thread whose first call is captured has no side stream yet (serial
    # launches); after an eager call it has one, and a new capture holds the
    # two branches; every replay gives the eager bits
    import threading
    cfg, dev, x, ids_d, w_d = _mixed_inputs(k3)
    ref = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2).cpu()
    torch.cuda.synchronize()
    errors = []

    def worker():
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
                ws = torch.empty(k3.moe_mxfp4_ffn_workspace_size(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k),
                                 dtype=torch.uint8, device="cuda")
            st.synchronize()
            for round_ in range(2):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=st):
                    k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2, out=out, workspace=ws)
                for _ in range(2):
                    out.fill_(float("nan"))
                    g.replay()
                    torch.cuda.synchronize()
                    assert torch.equal(out.cpu().view(torch.int32), ref.view(torch.int32)), f"capture {round_}"
                with torch.cuda.stream(st):  # eager: creates this thread's side stream
                    k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2, out=out, workspace=ws)
                st.synchronize()
                assert torch.equal(out.cpu().view(torch.int32), ref.view(torch.int32)), f"eager {round_}"
        except Exception as exc:
            errors.append(exc)

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert not errors, errors


@pytest.mark.parametrize(
    "E,k,D,I,T",
    # small-tile, streaming (grouped in the gate/up launch, x re-laid out first / read in place), large-tile, and
    # large-tile + streaming experts in one call (24 + 12: the streaming launches run on a side stream)
    [(8, 2, 128, 256, 64), (64, 4, 512, 512, 8), (64, 4, 512, 512, 3), (8, 2, 512, 512, 300),
     (40, 4, 512, 512, 90)],
)
def test_graph_replay_matches_eager(k3, E, k, D, I, T):
    # route + FFN captured into a HIP graph: every replay, with other eager work
    # in between, must reproduce the eager result bit for bit
    print(f"[ffn] graph replay E={E} k={k} D={D} I={I} T={T}", flush=True)
    cfg = moe_inputs.TINY.with_(E=E, k=k, D=D, I=I, T=T, config_id=43)
    batch = moe_inputs.make_batch(cfg)
    dev = device_experts(k3, cfg)
    x = bf16_dev(batch.x)
    z = torch.from_numpy(batch.z).cuda()
    b = torch.from_numpy(batch.b).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(k3.moe_mxfp4_ffn_workspace_size(T, D, I, E, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.float32, device="cuda")

    def step():
        k3.moe_route_topk(z, b, k, ids=ids, weights=w)
        k3.moe_mxfp4_ffn(x, ids, w, dev.w1, dev.w3, dev.w2, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.cpu().clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xA5)  # stale workspace contents must not matter
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.equal(got.view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("T,k", [(300, 2), (2048, 8)])  # 64- and 128-row down tiles
@pytest.mark.parametrize("e_lo,e_hi", [(96, 150), (70, 100)])
def test_large_tile_weights_fp16_cannot_hold(k3, e_lo, e_hi, T, k):
    # Large-tile shapes with w2 block exponents partly (96..150) or wholly
    # (70..100) outside the range whose values fp16 holds exactly: the down
    # product must redo those tiles with the exact bf16 pair, and h spans
    # magnitudes far from 1 (scaled per row and 256-feature slice).
    print(f"[ffn] large-tile exponents {e_lo}..{e_hi} T={T} k={k}", flush=True)
    cfg = moe_inputs.TINY.with_(E=8, k=k, D=512, I=512, T=T, e_lo=e_lo, e_hi=e_hi, config_id=60 + e_lo)
    got, ref, _, _ = small_case(k3, cfg)
    assert_ffn_close(got, ref, f"large-tile exponents {e_lo}..{e_hi}")


@pytest.mark.parametrize("T,k", [(300, 2), (2048, 8)])  # 64- and 128-row down tiles
@pytest.mark.parametrize("shift", [-40, 30])
def test_large_tile_extreme_activation_scale(k3, shift, T, k):
    # x scaled by 2^shift (exactly, in its bf16 exponent field): h lands far
    # outside fp16's range unless the per-slice scale follows it
    print(f"[ffn] large-tile x * 2^{shift} T={T} k={k}", flush=True)
    cfg = moe_inputs.TINY.with_(E=8, k=k, D=512, I=512, T=T, config_id=70)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    xb = batch.x.astype(np.int32)
    ex = (xb >> 7) & 0xFF
    assert ex.min() > max(0, -shift) and ex.max() < min(255, 255 - shift)  # no zero, no under/overflow
    x = ((xb & ~(0xFF << 7)) | ((ex + shift) << 7)).astype(np.uint16)
    dev = device_experts(k3, cfg)
    got = run_ffn(k3, dev, x, ids.astype(np.int32), w.astype(np.float32))
    ref = ffn_ref(x, ids, w, HostExperts(cfg))
    assert_ffn_close(got, ref, f"large-tile x * 2^{shift}")


class ScaledExperts:
    """Source-layout experts of `cfg` with the E8M0 bytes of the first 256
    intermediate features overridden: w1 / w3 rows 0..255 get `e_gu`, w2
    blocks 0..7 (columns 0..255) get `e_dn`."""

    def __init__(self, cfg, e_gu, e_dn):
        src = moe_inputs.ExpertSource(cfg)
        self.mats = []
        for e in range(cfg.E):
            (p1, s1), (p3, s3), (p2, s2) = src[e]
            s1, s3, s2 = s1.copy(), s3.copy(), s2.copy()
            s1[:256, :] = e_gu
            s3[:256, :] = e_gu
            s2[:, :8] = e_dn
            self.mats.append(((p1, s1), (p3, s3), (p2, s2)))

    def __getitem__(self, e):
        return self.mats[e]

    def __len__(self):
        return len(self.mats)

    def upload(self, k3, cfg):
        dev = {}
        for name, (shape, i) in {"w1": ((cfg.I, cfg.D), 0), "w3": ((cfg.I, cfg.D), 1), "w2": ((cfg.D, cfg.I), 2)}.items():
            t = torch.empty((cfg.E, shape[0], shape[1] // 32, 17), dtype=torch.uint8, device="cuda")
            for e in range(cfg.E):
                p, sc = self.mats[e][i]
                k3.mxfp4_tile(k3.mxfp4_repack(torch.from_numpy(p).cuda(), torch.from_numpy(sc).cuda()), out=t[e])
            dev[name] = t
        return dev


@pytest.mark.parametrize("e_gu,e_dn", [(114, 140), (80, 140)])
def test_large_tile_h_slices_far_apart(k3, e_gu, e_dn):
    # h of the first 256-wide slice about 2^-14 of the others' (rescaled sums
    # with factors near 2^14; through w2's large columns that slice makes
    # about 45% of the output) or about 2^-80 (a spread beyond the rescaling
    # span: the per-operand scaling path)
    cfg = moe_inputs.TINY.with_(E=4, k=2, D=512, I=512, T=300, config_id=48)
    print(f"[ffn] large-tile h slice scales e_gu={e_gu} e_dn={e_dn}", flush=True)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    ex = ScaledExperts(cfg, e_gu, e_dn)
    dev = ex.upload(k3, cfg)
    out = k3.moe_mxfp4_ffn(bf16_dev(batch.x), torch.from_numpy(ids.astype(np.int32)).cuda(),
                           torch.from_numpy(w.astype(np.float32)).cuda(), dev["w1"], dev["w3"], dev["w2"])
    ref = ffn_ref(batch.x, ids, w, ex)
    assert_ffn_close(out.cpu().numpy(), ref, f"e_gu={e_gu} e_dn={e_dn}")


def test_identity_weights_closed_form(k3):
    """W1 = W3 = [I; 0], W2 = 2^e [I | 0]: out[t] = sum_j w_j 2^(e_j) SiLU(x) x."""
    E, D, I, T, k = 4, 128, 256, 48, 2
    g = np.random.default_rng(12)

    def ident(rows, cols, p):
        codes = np.zeros((rows, cols), np.uint8)
        n = min(rows, cols)
        codes[np.arange(n), np.arange(n)] = 2
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), np.full((rows, cols // 32), 127 + p, np.uint8)

    w1 = k3.mxfp4_tile(torch.stack([k3.mxfp4_repack(*map(to_dev_u8, ident(I, D, 0))) for _ in range(E)]))
    w2 = k3.mxfp4_tile(torch.stack([k3.mxfp4_repack(*map(to_dev_u8, ident(D, I, e))) for e in range(E)]))
    x_bits = moe_inputs.bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    out = k3.moe_mxfp4_ffn(bf16_dev(x_bits), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                           w1, w1.clone(), w2).cpu().numpy()
    x = moe_inputs.bf16_to_f32(x_bits).astype(np.float64)
    base = x * x / (1.0 + np.exp(-x))
    expect = (w.astype(np.float64) * np.exp2(ids)).sum(axis=1, keepdims=True) * base
    assert_ffn_close(out, expect, "identity closed form")


def test_combine_large_batch_slot_batches(k3):
    # 8192 tokens x 32 threads: the combine takes its slots 8 at a time here;
    # k = 12 leaves a partial second batch (oracle on sampled tokens)
    cfg = moe_inputs.TINY.with_(E=16, k=12, D=512, I=512, T=8192, config_id=46)
    print(f"[ffn] combine slot batches T={cfg.T} k={cfg.k}", flush=True)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    dev = device_experts(k3, cfg)
    out = run_ffn(k3, dev, batch.x, ids.astype(np.int32), w.astype(np.float32))
    toks = np.array([0, 1, 4095, 5000, cfg.T - 1])
    ref = ffn_ref(batch.x, ids, w, HostExperts(cfg), tokens=toks)
    assert_ffn_close(out[toks], ref, f"tokens {toks.tolist()}")


# ---------------------------------------------------------------------------
# K3-shaped configs: all 896 experts resident on the device (15.7 GB; the
# session fixture k3_experts in conftest.py).


def last_tokens_of(ids, experts):
    """The largest token routed to each expert (its last grouped row)."""
    return [int(np.argwhere(ids == e)[:, 0].max()) for e in experts]


def covering_tokens(ids, experts):
    """A small set of tokens that together route to every expert listed (greedy cover)."""
    need = set(int(e) for e in experts)
    chosen = []
    while need:
        best = max(range(ids.shape[0]), key=lambda t: len(need & set(ids[t].tolist())))
        chosen.append(best)
        need -= set(ids[best].tolist())
    return chosen


def split_by_experts(ids, toks, parts):
    """Split the tokens into `parts` groups of about equal distinct-expert counts."""
    toks = sorted(set(int(t) for t in toks))
    total = len(np.unique(ids[toks]))
    groups, cur, seen = [], [], set()
    for t in toks:
        cur.append(t)
        seen |= set(ids[t].tolist())
        if len(seen) >= total / parts * (len(groups) + 1) and len(groups) < parts - 1:
            groups.append(cur)
            cur = []
    groups.append(cur)
    groups += [[] for _ in range(parts - len(groups))]
    return groups


def checked_tokens(name, ids, E):
    """Tokens of a K3 workload that the oracle checks, and why.

    decode: every token.  verify / prefill: the last token of every expert
    served by the large-tile kernels (more than 4 rows: its last row tile of
    both products) among the hottest (all of them at verify, the 8 hottest at
    prefill), and tokens covering every expert served by the weight-streaming
    kernels (at most 4 rows; at prefill at least one such expert).
    """
    T = ids.shape[0]
    if T <= 8:
        return list(range(T))
    counts = np.bincount(ids.reshape(-1), minlength=E)
    big = np.argsort(-counts, kind="stable")
    big = [int(e) for e in big if counts[e] > 4]
    stream = [int(e) for e in np.flatnonzero((counts > 0) & (counts <= 4))]
    if name == "prefill":
        big = big[:8]
        stream = stream[:1]
    return sorted(set(last_tokens_of(ids, big)) | set(covering_tokens(ids, stream)))


K3_PARTS = {"decode-t1": 1, "decode-t8": 4, "verify": 4, "prefill": 2}


@pytest.mark.parametrize("name,part", [(n, p) for n, c in K3_PARTS.items() for p in range(c)])
def test_k3_configs_end_to_end(k3, k3_experts, name, part):
    """GPU route -> GPU FFN at full size vs oracle route -> oracle FFN on the
    checked tokens (split into parts of about equal oracle cost)."""
    cfg = moe_inputs.CONFIGS[name]
    batch, x, z, b = moe_inputs.device.upload_batch(cfg)
    ids_d, w_d = k3.moe_route_topk(z, b, cfg.k)
    out = k3.moe_mxfp4_ffn(x, ids_d, w_d, k3_experts.w1, k3_experts.w3, k3_experts.w2).cpu().numpy()
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    assert np.all(np.isfinite(out))
    toks = split_by_experts(ids, checked_tokens(name, ids, cfg.E), K3_PARTS[name])[part]
    print(f"[ffn] K3 {name} T={cfg.T} part {part}: tokens {toks}", flush=True)
    assert toks
    ref = ffn_ref(batch.x, ids, w, batch.experts, tokens=np.array(toks))
    assert_ffn_close(out[toks], ref, f"{name} tokens {toks}")


def test_k3_checked_tokens_cover_every_tile_kind():
    # the token selection itself (host only): verify covers every expert of
    # either GEMM kind, prefill the 8 hottest experts' last rows and a
    # streaming expert
    for name in ("verify", "prefill"):
        cfg = moe_inputs.CONFIGS[name]
        batch = moe_inputs.make_batch(cfg)
        ids, _ = route_ref(batch.z, batch.b, cfg.k)
        toks = checked_tokens(name, ids, cfg.E)
        counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
        covered = set(ids[toks].reshape(-1).tolist())
        if name == "verify":
            assert covered >= set(np.flatnonzero(counts).tolist())
        hot = np.argsort(-counts, kind="stable")[:8]
        for e in hot:
            assert int(np.argwhere(ids == e)[:, 0].max()) in toks
        assert any(0 < counts[e] <= 4 for e in covered)
        parts = split_by_experts(ids, toks, K3_PARTS[name])
        assert sorted(t for p in parts for t in p) == sorted(set(toks)) and all(parts)


def test_k3_prefill_beyond_32bit_offsets(k3, k3_experts):
    """20000 tokens at K3 shape: more than (2^31 - 1) / (2 k max(D, I)) =
    18724 tokens, so the layer runs as a chunk of 18688 tokens and one of
    1312 with the large-tile and streaming kernels (there is no fallback
    path); the oracle checks the last rows of the hottest experts of each
    chunk, both sides of the chunk boundary and the last token."""
    cfg = moe_inputs.PREFILL.with_(T=20000, config_id=84)
    batch, x, z, b = moe_inputs.device.upload_batch(cfg)
    ids_d, w_d = k3.moe_route_topk(z, b, cfg.k)
    out = k3.moe_mxfp4_ffn(x, ids_d, w_d, k3_experts.w1, k3_experts.w3, k3_experts.w2).cpu().numpy()
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    assert np.all(np.isfinite(out))
    chunk = 18688
    toks = {chunk - 1, chunk, cfg.T - 1}
    for lo, hi in ((0, chunk), (chunk, cfg.T)):
        sub = ids[lo:hi]
        counts = np.bincount(sub.reshape(-1), minlength=cfg.E)
        for e in np.argsort(-counts, kind="stable")[:2]:
            toks.add(lo + int(np.argwhere(sub == e)[:, 0].max()))
    toks = sorted(toks)
    print(f"[ffn] K3 prefill T={cfg.T}: tokens {toks}", flush=True)
    ref = ffn_ref(batch.x, ids, w, batch.experts, tokens=np.array(toks))
    assert_ffn_close(out[toks], ref, f"T=20000 tokens {toks}")
