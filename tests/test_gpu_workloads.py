"""Full-size workloads, in the launch configuration the benchmark times,
checked against the oracle on sampled sequences.

  tiny     B=1,  M=4096,   H=8,  top-512, 64 blocks (both main-KV scale formats)
  full128  B=16, M=131072, H=64, top-512, 2048 blocks, 64 boosted rows/query
  step128  full128 shapes, 1 Full + 4 Reindex + 15 Reuse (20 attention calls)
  write1m  cache write 8192 tokens (m=2) + decode B=4 over M=524288
  stress   B=64, M=262144, full decoder step, clustered blocks and exact ties

Per sampled sequence: cache bytes identical to the oracle's quantisation;
Full-layer scores within tolerance, top-k and pool exact on the GPU's scores
and equal to the oracle's up to certified near-ties; every Reindex layer's
top-k likewise; attention of three layers within 1e-2 of the oracle.
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
from compressed_kv_cache_mxfp4_amd.decode_step import DecodeStep
import oracle
from gpu_common import (DEV, attn_close, brute_pool, brute_topk, build_gpu_cache, certify_topk,
                        oracle_cache_seq, say, score_close)

pytestmark = pytest.mark.gpu

SAMPLES = {"tiny": [0], "full128": [0, 15], "step128": [3], "write1m": [1], "stress": [0, 63], "enc128": [0, 9]}


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
    # Full-layer scores from the same launch configuration (only the score output pointer differs)
    q0, w0 = idx_qw[0]
    _, _, _, scores = K.index_full(cache["idx_codes"], cache["idx_scales"], lengths, q0, w0, k=wl.k,
                                   n_blocks=wl.n_blocks, return_scores=True)
    torch.cuda.synchronize()
    topk = [t.cpu().numpy() for t in step.topk]
    pool = step.pool.cpu().numpy()
    pool_len = step.pool_len.cpu().numpy()
    sched = step.schedule()
    certified = 0
    for b in SAMPLES[wl.name]:
        say(f"[{wl.name}] oracle on sequence {b}")
        ref = oracle_cache_seq(wl, b, fmt, cache)
        L = wl.cap
        qn = [(q.cpu().numpy()[b], w.cpu().numpy()[b]) for q, w in idx_qw]
        rt0, rpool, rpl, rs = oracle.index_full(ref["idx_codes"], ref["idx_scales"], L, qn[0][0], qn[0][1],
                                               wl.k, 8, wl.n_blocks)
        gs = scores[b].cpu().numpy()
        score_close(gs, rs)
        assert np.array_equal(topk[0][b], brute_topk(gs, wl.k))
        certified += certify_topk(topk[0][b], rt0, rs, wl.k)
        same_pool = False
        if wl.n_blocks > 0:
            bp, bpl, _ = brute_pool(gs, wl.n_blocks)
            assert pool_len[b] == bpl == rpl
            assert np.array_equal(pool[b], bp)
            _, _, rbs = brute_pool(rs, wl.n_blocks)
            certified += certify_topk(np.unique(pool[b][:bpl] // 8), np.unique(rpool[:rpl] // 8), rbs,
                                      wl.n_blocks)
            same_pool = np.array_equal(pool[b], rpool)
        ref_topk = [rt0]
        for i in range(1, 1 + wl.n_reindex):
            rti, rpsi = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, rpool, rpl, qn[i][0], qn[i][1], wl.k)
            ref_topk.append(rti)
            if same_pool:
                pos_scores = np.full(L, np.nan)
                pos_scores[rpool[:rpl]] = rpsi
                certified += certify_topk(topk[i][b], rti, pos_scores, wl.k)
        # attention: first, a Reindex-led and the last layer
        for j in sorted({0, min(1 + wl.reuse_per_index, step.n_attn - 1), step.n_attn - 1}):
            i = sched[j][1]
            ro, _ = oracle.attention(attn_q[j].cpu().numpy()[b], ref["main_codes"], ref["main_scales"], L, fmt,
                                     ref_topk[i], ref["main_codes"][L - 128:], ref["main_scales"][L - 128:], 128,
                                     1 / np.sqrt(512))
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
    say(f"[{wl.name}] certified near-tie index differences: {certified}")
    del cache, step
    torch.cuda.empty_cache()


def test_decode_step_graph_replay_matches_eager():
    """A step captured into a HIP graph reproduces the eager step bit for bit
    on every replay, with eager steps and host synchronisations in between."""
    wl = syn.small("graph", 41, B=3, cap=20000, H_idx=64, k=512, n_blocks=512, n_reindex=2,
                   reuse_per_index=2)
    say("[graph] capture and replay a 3 x 20000 decoder step")
    cache = build_gpu_cache(wl, 0)
    lengths = torch.tensor([20000, 19993, 7001], dtype=torch.int32, device=DEV)
    step = DecodeStep(cache, lengths, k=wl.k, n_blocks=wl.n_blocks, n_reindex=wl.n_reindex,
                      reuse_per_index=wl.reuse_per_index, main_fmt=0)
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


def test_step128_workload():
    _check_workload(syn.WORKLOADS["step128"], 1)


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
