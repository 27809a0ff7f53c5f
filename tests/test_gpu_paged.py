"""GPU parity of paged decoding (path_paged_decode_step, path_paged_import)
for a batch of sequences of different lengths, against the fp64 oracle: the
output of a step at position t of a sequence is row t of the walk over that
sequence's tokens, and after it the sequence's slots hold its keys carried to
t (oracle.transported_keys).

Each sequence is prefilled on its own (path_attn_fwd into a contiguous
cache, then path_paged_import into pages given by a shuffled page table), so
the paged kernels see scattered pages, ragged last pages and chunk edges."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check, check_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pa():
    import dependent_position_encoding_amd as pa
    pa.load_library()
    return pa


def _gather(pages, table, n):
    """Slots [0, n) of one sequence from [num_pages, H, P, ...] pages -> [H, n, ...]."""
    P = pages.shape[2]
    rows = [pages[int(table[j // P]), :, j % P] for j in range(n)]
    return torch.stack(rows, dim=1)


class Batch:
    """S sequences with their own token streams, prefilled to lens[s] tokens
    into a shared paged cache."""

    def __init__(self, wl, lens, steps, page_size, k_dtype, seed, spare_pages=7, device="cpu"):
        pa = _pa()
        self.pa, self.wl, self.lens, self.steps = pa, wl, list(lens), steps
        S, H, d = len(lens), wl.H, wl.d
        self.P = page_size
        self.max_keys = max(lens) + steps
        self.stride = (self.max_keys + page_size - 1) // page_size
        need = [(n + steps + page_size - 1) // page_size for n in lens]
        num_pages = sum(need) + spare_pages
        perm = np.random.default_rng(seed).permutation(num_pages)
        table = np.full((S, self.stride), -1, dtype=np.int32)
        at = 0
        for s in range(S):
            table[s, :need[s]] = perm[at:at + need[s]]
            at += need[s]
        self.table_np = table
        self.table = torch.from_numpy(table).to(DEV)
        self.cache = pa.PagedCache(num_pages, page_size, H, d, dtype=wl.dtype, k_dtype=k_dtype,
                                   gate=wl.fox, device=DEV)
        self.x = [workloads.make_inputs(wl.replace(N=1), device=device, variant=seed * 31 + s,
                                        L=lens[s] + steps) for s in range(S)]
        for s in range(S):
            n = lens[s]
            if n == 0:
                continue
            g = {k: (v[:, :, :n].contiguous().to(DEV) if v is not None else None)
                 for k, v in self.x[s].items()}
            src = pa.Cache(1, H, n, d, dtype=wl.dtype, k_dtype=k_dtype, gate=wl.fox, device=DEV)
            pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"], scale=wl.scale,
                   cache=src)
            pa.paged_import(src, self.cache, self.table[s:s + 1].contiguous(),
                            torch.tensor([n], dtype=torch.int32, device=DEV), self.max_keys)
        self.seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)

    def token(self, i):
        """Inputs of step i for every sequence, [S, H, d] / [S, H]."""
        out = {}
        for name in ("q", "k", "v", "w", "beta", "logf"):
            if self.x[0][name] is None:
                out[name] = None
                continue
            out[name] = torch.cat([x[name][:, :, n + i] for x, n in zip(self.x, self.lens)],
                                  dim=0).contiguous().to(DEV)
        return out

    def step(self, i, out=None):
        t = self.token(i)
        return self.pa.paged_decode_step(self.cache, self.table, self.seq_lens, self.max_keys,
                                         t["q"], t["k"], t["v"], t["w"], t["beta"], t["logf"],
                                         scale=self.wl.scale, out=out)


def _run_and_check(b: Batch, bf16: bool, k_dtype):
    outs = [b.step(i) for i in range(b.steps)]
    torch.cuda.synchronize()
    assert b.seq_lens.cpu().tolist() == [n + b.steps for n in b.lens]
    H = b.wl.H
    for s in range(len(b.lens)):
        n = b.lens[s]
        print(f"  sequence {s}: {n} cached keys, page {b.P}", flush=True)
        go = np.stack([workloads.as_slices_f64(o[s:s + 1]) for o, _ in outs], axis=1)
        gl = np.stack([workloads.as_slices_f64(l[s:s + 1]) for _, l in outs], axis=1)
        f64 = {k: (workloads.as_slices_f64(v) if v is not None else None)
               for k, v in b.x[s].items()}
        ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"],
                                 f64["logf"], b.wl.scale, rows=np.arange(n, n + b.steps))
        check(f"paged o (seq {s})", go, ro, bf16=bf16)
        check(f"paged lse (seq {s})", gl, rl, bf16=bf16)
        rk = oracle.transported_keys(f64["k"], f64["w"], f64["beta"], n + b.steps - 1)
        kc = _gather(b.cache.kpages, b.table_np[s], n + b.steps)        # [H, n+steps, d]
        check_cache(f"paged keys (seq {s})", workloads.as_slices_f64(kc[None]), rk, k_dtype,
                    b.steps)
        # values are copied exactly
        vc = _gather(b.cache.vpages, b.table_np[s], n + b.steps).cpu()
        assert torch.equal(vc, b.x[s]["v"][0, :, :n + b.steps].to(vc.dtype))
        if b.cache.gpages is not None:
            gc = _gather(b.cache.gpages, b.table_np[s], n + b.steps).cpu().double().numpy()
            lf = b.x[s]["logf"][0].double().numpy()[:, :n + b.steps]
            np.testing.assert_allclose(gc, np.cumsum(lf, axis=1), rtol=1e-4, atol=1e-3)
        assert H == kc.shape[0]


@pytest.mark.parametrize("page_size", [16, 64, 128])
def test_paged_bf16_mixed_lengths(page_size):
    # empty, one key, a page edge, a chunk edge, ragged tails across chunks
    wl = workloads.CONFIGS["fox"].replace(H=2)
    lens = [0, 1, page_size, 128, 257, 700]
    b = Batch(wl, lens, steps=3, page_size=page_size, k_dtype=torch.bfloat16, seed=page_size)
    _run_and_check(b, True, torch.bfloat16)


@pytest.mark.parametrize("gate", [False, True])
def test_paged_fp32(gate):
    wl = workloads.CONFIGS["fox"].replace(H=2, d=32, dtype=torch.float32, fox=gate,
                                          scale=32 ** -0.5)
    b = Batch(wl, [5, 0, 190, 64], steps=2, page_size=32, k_dtype=torch.float32, seed=3)
    _run_and_check(b, False, torch.float32)


def test_paged_bf16_head_dim_32_no_gate():
    wl = workloads.CONFIGS["fox"].replace(H=2, d=32, fox=False, scale=32 ** -0.5)
    b = Batch(wl, [3, 128, 300], steps=2, page_size=32, k_dtype=torch.bfloat16, seed=5)
    _run_and_check(b, True, torch.bfloat16)


def test_paged_bf16_fp32_keys_head_dim_16():
    wl = workloads.CONFIGS["fox"].replace(H=3, d=16, scale=0.25)
    b = Batch(wl, [33, 130], steps=2, page_size=16, k_dtype=torch.float32, seed=4)
    _run_and_check(b, True, torch.float32)


def test_paged_matches_contiguous_step_bitwise():
    """Same prefill, same tokens: the paged step and the contiguous fused step
    run the same per-chunk arithmetic, so outputs and caches agree exactly."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=3, H=2)
    L, steps, P = 300, 3, 64
    x = workloads.make_inputs(wl, device="cpu", variant=11, L=L + steps)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    cont = pa.Cache(3, 2, L + steps, wl.d, dtype=wl.dtype, gate=True, device=DEV)
    pre = lambda n: g[n][:, :, :L].contiguous()
    pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"), logf=pre("logf"),
           scale=wl.scale, cache=cont)
    stride = (L + steps + P - 1) // P
    perm = np.random.default_rng(5).permutation(3 * stride + 2)[:3 * stride].reshape(3, stride)
    table = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    paged = pa.PagedCache(3 * stride + 2, P, 2, wl.d, dtype=wl.dtype, gate=True, device=DEV)
    seq = torch.full((3,), L, dtype=torch.int32, device=DEV)
    pa.paged_import(cont, paged, table, seq, L + steps)
    tok = lambda n, t: g[n][:, :, t].contiguous()
    for t in range(L, L + steps):
        args = [tok(n, t) for n in ("q", "k", "v", "w", "beta", "logf")]
        oc, lc = pa.decode_step(cont, t, *args, scale=wl.scale)
        op, lp = pa.paged_decode_step(paged, table, seq, L + steps, *args, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(oc, op) and torch.equal(lc, lp), t
    for s in range(3):
        kc = _gather(paged.kpages, perm[s], L + steps)
        assert torch.equal(kc, cont.kcache[s, :, :L + steps])
    assert seq.cpu().tolist() == [L + steps] * 3


def test_paged_bad_entries_give_nan_without_touching_others():
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(H=2)
    b = Batch(wl, [100, 200, 50, 128], steps=1, page_size=64, k_dtype=torch.bfloat16, seed=9)
    keys_before = b.cache.kpages.clone()
    # sequence 1: its second page entry points past the pool; sequence 2: a
    # length beyond max_keys; sequence 3: the page of slot t - 1 (whose gate
    # prefix every chunk reads; the new token at t = 128 opens the next page)
    # is negative
    b.table[1, 1] = b.cache.num_pages + 3
    b.seq_lens[2] = b.max_keys
    b.table[3, 1] = -2
    o, lse = b.step(0)
    torch.cuda.synchronize()
    for s in (1, 2, 3):
        assert torch.isnan(o[s]).all() and torch.isnan(lse[s]).all(), s
    assert torch.isfinite(o[0]).all() and torch.isfinite(lse[0]).all()
    assert b.seq_lens.cpu().tolist() == [101, 201, b.max_keys, 129]
    # sequences 2 and 3 wrote nothing; sequence 0 is right
    for s in (2, 3):
        ts = b.table_np[s]
        for p in ts[ts >= 0]:
            assert torch.equal(b.cache.kpages[int(p)], keys_before[int(p)]), s
    f64 = {k: (workloads.as_slices_f64(v) if v is not None else None) for k, v in b.x[0].items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=[100])
    check("paged o (seq 0, others bad)", workloads.as_slices_f64(o[0:1])[:, None], ro, bf16=True)


def test_paged_step_graph_replay():
    """One captured step replayed for successive positions (seq_lens advances
    on the device), with the next token copied into the captured input
    buffers between replays; every replay against the oracle."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(H=2)
    steps = 4
    b = Batch(wl, [70, 129, 10], steps=steps, page_size=32, k_dtype=torch.bfloat16, seed=21)
    bufs = b.token(0)
    o = torch.empty_like(bufs["q"])
    lse = torch.empty(bufs["beta"].shape, dtype=torch.float32, device=DEV)
    ws = torch.empty(pa.paged_decode_workspace_bytes(3, wl.H, wl.d, wl.dtype, b.max_keys),
                     dtype=torch.uint8, device=DEV)

    def launch():
        pa.paged_decode_step(b.cache, b.table, b.seq_lens, b.max_keys, bufs["q"], bufs["k"],
                             bufs["v"], bufs["w"], bufs["beta"], bufs["logf"], scale=wl.scale,
                             workspace=ws, out=(o, lse))

    # capture on a side stream; the capture itself does not execute
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            launch()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    got_o, got_l = [], []
    for i in range(steps):
        nxt = b.token(i)
        for k in bufs:
            if bufs[k] is not None:
                bufs[k].copy_(nxt[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o.append(o.clone())
        got_l.append(lse.clone())
    assert b.seq_lens.cpu().tolist() == [n + steps for n in b.lens]
    for s in range(3):
        n = b.lens[s]
        f64 = {k: (workloads.as_slices_f64(v) if v is not None else None)
               for k, v in b.x[s].items()}
        ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"],
                                 f64["logf"], wl.scale, rows=np.arange(n, n + steps))
        go = np.stack([workloads.as_slices_f64(x[s:s + 1]) for x in got_o], axis=1)
        gl = np.stack([workloads.as_slices_f64(x[s:s + 1]) for x in got_l], axis=1)
        check(f"graph paged o (seq {s})", go, ro, bf16=True)
        check(f"graph paged lse (seq {s})", gl, rl, bf16=True)


def test_paged_serving_shape_sampled():
    """The paged step at the shape the benchmark times: 32 sequences x 32
    heads, d = 64, bf16 with the gate, cached lengths uniform in [1024, 8192]
    (the benchmark's seed), page size 64; every sequence prefilled and
    imported, two fused steps, and the outputs of sampled (sequence, head)
    slices against the oracle's rows."""
    import numpy as np
    rng = np.random.default_rng(7)
    lens = [int(n) for n in rng.integers(1024, 8193, size=32)]
    wl = workloads.CONFIGS["fox"].replace(H=32)
    print(f"case paged serving shape, lengths {min(lens)}..{max(lens)}", flush=True)
    b = Batch(wl, lens, steps=2, page_size=64, k_dtype=torch.bfloat16, seed=13, device=DEV)
    outs = [b.step(i) for i in range(2)]
    torch.cuda.synchronize()
    assert b.seq_lens.cpu().tolist() == [n + 2 for n in lens]
    for s in (0, 13, 31):
        n = lens[s]
        for h in (0, 17):
            f64 = {k: (workloads.as_slices_f64(v, heads=[h]) if v is not None else None)
                   for k, v in b.x[s].items()}
            ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"],
                                     f64["logf"], wl.scale, rows=np.arange(n, n + 2))
            go = np.stack([workloads.as_slices_f64(o[s:s + 1, h:h + 1]) for o, _ in outs], axis=1)
            gl = np.stack([workloads.as_slices_f64(l[s:s + 1, h:h + 1]) for _, l in outs], axis=1)
            check(f"paged o (seq {s}, {n} keys, head {h})", go, ro, bf16=True)
            check(f"paged lse (seq {s}, head {h})", gl, rl, bf16=True)
