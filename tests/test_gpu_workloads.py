"""Full-size workloads, in the launch configuration the benchmark times,
checked against the oracle on sampled sequences.

  tiny     B=1,  M=4096,   H=8,  top-512, 64 blocks (both main-KV scale formats)
  full128  B=16, M=131072, H=64, top-512, 2048 blocks, 64 boosted rows/query
  step128  full128 shapes, 1 Full + 4 Reindex + 15 Reuse (20 attention calls),
           with both main-KV scale formats (E8M0 is the benchmarked one)
  write1m  cache write 8192 tokens (m=2) + decode B=4 over M=524288
  stress   B=64, M=262144, full decoder step, clustered blocks and exact ties

The scorer and both attention kernels place sequence b on XCD b mod 8 when the
batch is a multiple of 8, so the batched workloads sample one sequence of each
residue b mod 8.  Per sampled sequence: indexer-K bytes identical to the
oracle's quantisation (main-KV bytes on the rows attention reads); Full-layer
scores within tolerance, top-k and pool exact on the GPU's own scores and
equal to the oracle's up to certified near-ties; every Reindex layer's pool
scores within tolerance, its top-k exact on the GPU's own pool scores and
equal to the oracle's up to certified near-ties -- against the oracle run on
the GPU's own pool when the two pools differ by a near-tie; attention of three
layers within 1e-2 of the oracle.  The counts of certified near-ties are
printed.
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
from compressed_kv_cache_mxfp4_amd.decode_step import DecodeStep
import oracle
from gpu_common import (DEV, attn_close, brute_pool, brute_topk, build_gpu_cache, certify_topk,
                        oracle_cache_seq, oracle_main_rows, remap_positions, say, score_close)

pytestmark = pytest.mark.gpu

_XCD8_16 = [0, 9, 2, 11, 4, 13, 6, 15]            # b mod 8 = 0..7 among 16 sequences
_XCD8_64 = [0, 9, 18, 27, 36, 45, 54, 63]         # b mod 8 = 0..7 among 64 sequences
SAMPLES = {"tiny": [0], "full128": _XCD8_16, "step128": _XCD8_16, "write1m": [0, 3], "stress": _XCD8_64,
           "enc128": [0, 9]}


def _inputs(wl):
    n_idx = 1 + wl.n_reindex
    idx_qw = [(syn.index_query(wl, i, DEV), syn.index_weights(wl, i, DEV)) for i in range(n_idx)]
    attn_q = [syn.attn_query(wl, j, DEV) for j in range(wl.n_attn_calls)]
    return idx_qw, attn_q


def _check_workload(wl, fmt):
    say(f"[{wl.name}] building B={wl.B} M={wl.cap} cache on the GPU (fmt {fmt})")
    cache = build_gpu_cache(wl, fmt)
    lengths = torch.full((wl.B,), wl.cap, dtype=torch.int32, device=DEV)
    step = DecodeStep(cache, lengths, k=wl.k, n_blocks=wl.n_blocks, n_reindex=wl.n_reindex,
                      reuse_per_index=wl.reuse_per_index, main_fmt=fmt)
    idx_qw, attn_q = _inputs(wl)
    step.run(idx_qw, attn_q)
    # Scores of every index layer from the same launch configuration (only
    # the score output pointer differs); the selections must be the step's.
    q0, w0 = idx_qw[0]
    t0, _, _, scores = K.index_full(cache["idx_codes"], cache["idx_scales"], lengths, q0, w0, k=wl.k,
                                    n_blocks=wl.n_blocks, return_scores=True)
    pool_scores = [None]
    for i in range(1, 1 + wl.n_reindex):
        qi, wi = idx_qw[i]
        ti, psi = K.index_pool(cache["idx_codes"], cache["idx_scales"], lengths, step.pool, step.pool_len, qi, wi,
                               k=wl.k, return_scores=True)
        assert torch.equal(ti, step.topk[i]), f"Reindex layer {i}: rerun with a score output differs"
        pool_scores.append(psi.cpu().numpy())
    assert torch.equal(t0, step.topk[0]), "Full layer: rerun with a score output differs"
    torch.cuda.synchronize()
    topk = [t.cpu().numpy() for t in step.topk]
    pool = step.pool.cpu().numpy()
    pool_len = step.pool_len.cpu().numpy()
    sched = step.schedule()
    cert = dict(full=0, blocks=0, reindex=0)
    pools_differ = 0
    L = wl.cap
    for b in SAMPLES[wl.name]:
        say(f"[{wl.name}] oracle on sequence {b} (XCD residue {b % 8})")
        ref = oracle_cache_seq(wl, b, fmt, cache, need_main=False)
        qn = [(q.cpu().numpy()[b], w.cpu().numpy()[b]) for q, w in idx_qw]
        rt0, rpool, rpl, rs = oracle.index_full(ref["idx_codes"], ref["idx_scales"], L, qn[0][0], qn[0][1],
                                               wl.k, 8, wl.n_blocks)
        gs = scores[b].cpu().numpy()
        score_close(gs, rs)
        assert np.array_equal(topk[0][b], brute_topk(gs, wl.k))
        cert["full"] += certify_topk(topk[0][b], rt0, rs, wl.k)
        if wl.n_blocks > 0:
            bp, bpl, _ = brute_pool(gs, wl.n_blocks)
            assert pool_len[b] == bpl == rpl
            assert np.array_equal(pool[b], bp)
            _, _, rbs = brute_pool(rs, wl.n_blocks)
            cert["blocks"] += certify_topk(np.unique(pool[b][:bpl] // 8), np.unique(rpool[:rpl] // 8), rbs,
                                           wl.n_blocks)
            if not np.array_equal(pool[b], rpool):
                pools_differ += 1
        ref_topk = [rt0]
        n = int(pool_len[b])
        gpool = pool[b][:n]
        for i in range(1, 1 + wl.n_reindex):
            # the oracle rescoring the GPU's own pool (equal to the oracle's
            # pool unless a certified near-tie moved a block)
            rti, rpsi = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, pool[b], n, qn[i][0], qn[i][1],
                                          wl.k)
            gps = pool_scores[i][b][:n]
            score_close(gps, rpsi)
            assert np.array_equal(topk[i][b], brute_topk(gps, wl.k, gpool)), f"Reindex layer {i} selection"
            pos_scores = np.full(L, np.nan)
            pos_scores[gpool] = rpsi
            cert["reindex"] += certify_topk(topk[i][b], rti, pos_scores, wl.k)
            ref_topk.append(rti)
        # attention: first, a Reindex-led and the last layer
        layers = sorted({0, min(1 + wl.reuse_per_index, step.n_attn - 1), step.n_attn - 1})
        need = set(range(L - 128, L))
        for j in layers:
            i = sched[j][1]
            need |= {int(p) for p in ref_topk[i] if p >= 0} | {int(p) for p in topk[i][b] if p >= 0}
        rows = np.array(sorted(need), np.int64)
        mc, ms = oracle_main_rows(wl, b, fmt, cache, rows)
        win = remap_positions(np.arange(L - 128, L), rows)
        for j in layers:
            i = sched[j][1]
            ro, _ = oracle.attention(attn_q[j].cpu().numpy()[b], mc, ms, len(rows), fmt,
                                     remap_positions(ref_topk[i], rows), mc[win], ms[win], 128, 1 / np.sqrt(512))
            if set(topk[i][b].tolist()) == set(ref_topk[i].tolist()):
                got = step.out[j][b:b + 1].cpu()
            else:  # near-tie selections differ: attend the oracle's selection on the GPU
                got = K.sparse_attn_decode(attn_q[j][b:b + 1], cache["main_codes"][b:b + 1],
                                           cache["main_scales"][b:b + 1], lengths[b:b + 1],
                                           torch.from_numpy(ref_topk[i][None]).to(DEV), fmt,
                                           swa_codes=cache["main_codes"][b:b + 1],
                                           swa_scales=cache["main_scales"][b:b + 1],
                                           swa_len=torch.full((1,), 128, dtype=torch.int32, device=DEV),
                                           swa_stride=L, swa_cap=128, swa_row0=L - 128).cpu()
            worst = attn_close(got, ro[None])
            say(f"[{wl.name}] seq {b} attention layer {j}: worst rel err {worst:.2e}")
    say(f"[{wl.name}] certified near-tie index differences: top-k {cert['full']}, pool blocks {cert['blocks']}, "
        f"Reindex {cert['reindex']}; sequences whose pool differs from the oracle's: {pools_differ}")
    del cache, step
    torch.cuda.empty_cache()


def test_decode_step_graph_replay_matches_eager():
    """A step captured into a HIP graph reproduces the eager step bit for bit
    on every replay, with eager steps and host synchronisations in between."""
    wl = syn.small("graph", 41, B=3, cap=20000, H_idx=64, k=512, n_blocks=512, n_reindex=2,
                   reuse_per_index=2)
    say("[graph] capture and replay a 3 x 20000 decoder step")
    cache = build_gpu_cache(wl, 0)
    lens = [20000, 19993, 7001]
    lengths = torch.tensor(lens, dtype=torch.int32, device=DEV)
    # each sequence's window: its own last 128 visible entries, in a buffer of their own
    swa = dict(codes=torch.stack([cache["main_codes"][b, L - 128:L] for b, L in enumerate(lens)]).contiguous(),
               scales=torch.stack([cache["main_scales"][b, L - 128:L] for b, L in enumerate(lens)]).contiguous(),
               row0=0, stride=128, length=torch.full((3,), 128, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        DecodeStep(cache, lengths, k=wl.k, n_blocks=wl.n_blocks, n_reindex=wl.n_reindex,
                   reuse_per_index=wl.reuse_per_index, main_fmt=0)
    step = DecodeStep(cache, lengths, k=wl.k, n_blocks=wl.n_blocks, n_reindex=wl.n_reindex,
                      reuse_per_index=wl.reuse_per_index, main_fmt=0, swa=swa)
    idx_qw, attn_q = _inputs(wl)

    def snapshot():
        torch.cuda.synchronize()
        return ([t.clone() for t in step.topk], step.pool.clone(), step.pool_len.clone(),
                [o.clone() for o in step.out])

    def same(a, b):
        return (all(torch.equal(x, y) for x, y in zip(a[0], b[0])) and torch.equal(a[1], b[1])
                and torch.equal(a[2], b[2]) and all(torch.equal(x, y) for x, y in zip(a[3], b[3])))

    step.run(idx_qw, attn_q)
    ref = snapshot()
    graph = step.capture(idx_qw, attn_q)
    for rep in range(3):
        # clobber the outputs, replay, compare; then an eager step in between
        for t in step.topk:
            t.fill_(-7)
        for o in step.out:
            o.fill_(0)
        graph.replay()
        assert same(snapshot(), ref), f"replay {rep} differs from the eager step"
        step.run(idx_qw, attn_q)
        assert same(snapshot(), ref), f"eager step after replay {rep} differs"
    # the completion counters of the attention workspace are back at zero
    assert int(step.ws_attn[:65536 * 4].count_nonzero()) == 0  # CSA2_ATTN_WS_COUNTER_BYTES
    del graph, step, cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [0, 1])
def test_tiny_workload(fmt):
    _check_workload(syn.WORKLOADS["tiny"], fmt)


def test_full128_workload():
    _check_workload(syn.WORKLOADS["full128"], 0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_step128_workload(fmt):
    # fmt 0 (E8M0 main-KV scales) is the configuration the benchmark times
    _check_workload(syn.WORKLOADS["step128"], fmt)


def test_write1m_workload():
    wl = syn.WORKLOADS["write1m"]
    say("[write1m] cache write 8192 tokens, m=2")
    lat, gate, w = syn.write_inputs(wl, DEV)
    got = K.cache_write(lat, gate, 2, w, 0)
    torch.cuda.synchronize()
    ref = oracle.cache_write(lat.cpu().numpy(), gate.cpu().numpy(), 2, w.cpu().numpy(), 0)
    from test_gpu_attention import _certified_code_mismatch
    g = {k_: v.cpu().numpy() for k_, v in got.items()}
    nm = _certified_code_mismatch(ref["y"], ref["main_codes"], ref["main_scales"], g["main_codes"], g["main_scales"], 16, 0)
    nk = _certified_code_mismatch(ref["k"], ref["idx_codes"], ref["idx_scales"], g["idx_codes"], g["idx_scales"], 32, 0)
    say(f"[write1m] certified byte differences: main {nm}, indexer {nk}")
    _check_workload(wl, 0)


def test_stress_workload():
    _check_workload(syn.WORKLOADS["stress"], 0)


def test_enc128_workload():
    # encoder source layer: m = 2 entries, no candidate pool
    _check_workload(syn.WORKLOADS["enc128"], 0)
