"""Graph-padded calls under HIP graph capture.

"[GDN] Spec-decoding-aware attention kernel" ("Related issues") names the
size(0) == num_actual_tokens precondition that breaks graph capture, and the
graph-padded spec metadata is named on "[XE2] Support MTP of QWEN model".
Reading: a step is captured once at padded shapes (scalars are frozen in the
graph) and replayed with batches of fewer real rows.  Pad rows carry NULL (0)
slots and their tokens sit in rows past the real ones, so they read and write
no pool; the real rows must equal an eager call on the unpadded batch bit for
bit, replay after replay, with eager work between the replays.  Prefill rows
keep a fixed row count and token budget: the last prefill row is a pad row
that takes the tokens the real rows leave over."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import helpers
import synth
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, bf, cfg_of, f32,
                            gpu_available, i32, say, u8)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]

Hk, Hv, DK, K, SLOTS = 4, 8, 128, 3, 96
NS_PAD, ND_PAD = 8, 6
NP_PAD, PF_TOK = 3, 200  # prefill rows (the last one pads) and their token budget


def scenario(seed, ns, nd, pf=None, ns_pad=NS_PAD, num_slots=SLOTS, k=K, heads=(Hk, Hv)):
    """Padded metadata for ns real spec rows of k tokens (of ns_pad), nd real
    decodes and (with pf, a list of at most NP_PAD - 1 lengths) real prefill
    rows, and the unpadded case with the same real rows."""
    NS_PAD, SLOTS, K = ns_pad, num_slots, k  # noqa: N806 (the pads of this scenario)
    Hk, Hv = heads  # noqa: N806
    rng = np.random.default_rng(seed)
    pf = None if pf is None else list(pf)
    npf, pf_real = (0, 0) if pf is None else (NP_PAD, sum(pf))
    pf_tok = PF_TOK if pf is not None else 0
    t_pad = ND_PAD + pf_tok + NS_PAD * K
    t_real = nd + pf_real + ns * K
    case = helpers.small_case(seed=seed, Hk=Hk, Hv=Hv, dk=DK, dv=DK, K=K, T=t_pad,
                              num_slots=SLOTS)
    n_pf_rows = 0 if pf is None else len(pf)
    slots = rng.choice(np.arange(1, SLOTS), ns * K + nd + n_pf_rows,
                       replace=False).astype(np.int32)
    rows = rng.permutation(t_real).astype(np.int32)      # real tokens -> rows [0, t_real)
    pad_rows = np.arange(t_real, t_pad, dtype=np.int32)  # pad tokens -> rows past them
    spec_rows, dec_rows, pf_rows = rows[:ns * K], rows[ns * K:ns * K + nd], rows[ns * K + nd:]
    spec_pad = pad_rows[:(NS_PAD - ns) * K]
    dec_pad = pad_rows[(NS_PAD - ns) * K:(NS_PAD - ns) * K + ND_PAD - nd]
    pf_pad = pad_rows[(NS_PAD - ns) * K + ND_PAD - nd:]
    # spec rows
    ssi = np.zeros((NS_PAD, K), np.int32)
    ssi[:ns] = slots[:ns * K].reshape(ns, K)
    nacc = np.ones(NS_PAD, np.int32)
    nacc[:ns] = rng.integers(1, K + 1, ns)
    sqsl = np.arange(0, NS_PAD * K + 1, K, dtype=np.int32)
    stix = np.concatenate([spec_rows, spec_pad]).astype(np.int32)
    # non-spec rows: decodes, then the prefill rows (real ones, empty pads,
    # and a last pad row holding the tokens left over)
    nrows = ND_PAD + npf
    cache = np.zeros(nrows, np.int32)
    cache[:nd] = slots[ns * K:ns * K + nd]
    cache[ND_PAD:ND_PAD + n_pf_rows] = slots[ns * K + nd:]
    his = np.zeros(nrows, np.uint8)
    his[:nd] = rng.integers(0, 2, nd)
    his[ND_PAD:ND_PAD + n_pf_rows] = rng.integers(0, 2, n_pf_rows)
    lens = [1] * ND_PAD
    if pf is not None:
        lens += pf + [0] * (NP_PAD - 1 - len(pf)) + [PF_TOK - pf_real]
    dqsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dtix = np.concatenate([dec_rows, dec_pad, pf_rows, pf_pad]).astype(np.int32)
    padded = dict(sqsl=sqsl, ssi=ssi, nacc=nacc, stix=stix, dqsl=dqsl, cache=cache, his=his,
                  dtix=dtix, t=t_pad, npf=npf, pf_tok=pf_tok, ns_pad=NS_PAD, k=K)
    real = dict(case)
    for k in ("mixed_qkv", "a", "b"):
        real[k] = case[k][:t_real]
    real["num_actual_tokens"] = t_real
    real["spec"] = (helpers.spec_meta(sqsl[:ns + 1], ssi[:ns], nacc[:ns], stix[:ns * K])
                    if ns else None)
    rl = [1] * nd + ([] if pf is None else pf)
    rc = np.concatenate([cache[:nd], cache[ND_PAD:ND_PAD + n_pf_rows]])
    rh = np.concatenate([his[:nd], his[ND_PAD:ND_PAD + n_pf_rows]])
    rt = np.concatenate([dec_rows, pf_rows]).astype(np.int32)
    real["nonspec"] = (helpers.nonspec_meta(rl, rc, his=rh, tix=rt, num_decodes=nd)
                       if rl else None)
    return case, padded, real


class Static:
    """Device buffers a captured step reads and writes (fixed addresses)."""

    def __init__(self, case, padded, with_decodes):
        self.g = Gpu(case)
        self.cfg = cfg_of(case)
        self.meta = {k: (i32(v) if v.dtype == np.int32 else u8(v))
                     for k, v in padded.items() if isinstance(v, np.ndarray)}
        self.t, self.npf, self.pf_tok = padded["t"], padded["npf"], padded["pf_tok"]
        self.ns_pad, self.k = padded["ns_pad"], padded["k"]
        self.with_decodes = with_decodes
        self.ws = None
        if self.npf:
            import speculative_decoding_causal_amd as gdn
            d = case["dims"]
            nbytes = gdn.gdn_workspace_bytes(self.cfg, d["L"], d["num_slots"],
                                             ND_PAD + self.pf_tok, self.npf)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def load(self, case, padded):
        g = self.g
        for name, t, src in (("qkv", g.qkv, case["mixed_qkv"]), ("a", g.a, case["a"]),
                             ("b", g.b, case["b"]), ("w", g.w, case["conv_weight"]),
                             ("conv", g.conv, case["conv_state"])):
            t.copy_(bf(src))
        g.A_log.copy_(f32(case["A_log"]))
        g.dt_bias.copy_(f32(case["dt_bias"]))
        g.ssm.copy_(f32(case["ssm_state"]))
        for k, t in self.meta.items():
            t.copy_(i32(padded[k]) if padded[k].dtype == np.int32 else u8(padded[k]))
        assert (padded["npf"], padded["pf_tok"]) == (self.npf, self.pf_tok)

    def call(self):
        import speculative_decoding_causal_amd as gdn
        g, m = self.g, self.meta
        ts = self.ns_pad * self.k
        spec = dict(spec_query_start_loc=m["sqsl"], spec_state_indices=m["ssi"],
                    num_accepted_tokens=m["nacc"], spec_token_indx=m["stix"],
                    num_spec_tokens=ts)
        if not self.with_decodes:
            gdn.gdn_spec_attention(self.cfg, g.qkv[:ts], g.a[:ts], g.b[:ts], g.w, None, g.A_log,
                                   g.dt_bias, g.conv, g.ssm, m["sqsl"], m["ssi"], m["nacc"],
                                   g.out, spec_token_indx=m["stix"], num_spec_tokens=ts,
                                   num_actual_tokens=ts, conv_turns=g.turns)
        else:
            gdn.gdn_attention(self.cfg, g.qkv, g.a, g.b, g.w, None, g.A_log, g.dt_bias, g.conv,
                              g.ssm, g.out, num_decodes=ND_PAD, num_prefills=self.npf,
                              num_non_spec_tokens=ND_PAD + self.pf_tok,
                              query_start_loc=m["dqsl"],
                              non_spec_state_indices=m["cache"], has_initial_state=m["his"],
                              non_spec_token_indx=m["dtix"], num_actual_tokens=self.t,
                              workspace=self.ws, conv_turns=g.turns, **spec)


def _run_graph(with_decodes, plan, **pads):
    case0, pad0, _ = scenario(*plan[0], **pads)
    st = Static(case0, pad0, with_decodes)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.call()                       # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.call()
    for step in plan:
        seed, ns, nd = step[:3]
        case, padded, real = scenario(*step, **pads)
        st.load(case, padded)
        torch.cuda.synchronize()
        pf = f", prefills {step[3]}" if len(step) > 3 else ""
        say(f"graph replay: {ns} spec rows, {nd} decodes{pf} "
            f"(padded to {padded['ns_pad']}, {ND_PAD})")
        graph.replay()
        torch.cuda.synchronize()
        if st.g.turns is not None:
            assert int(st.g.turns.abs().sum().item()) == 0, "turn counters not back at 0"
        eager = Gpu(real)
        if with_decodes:
            eager.attention()
        else:
            eager.spec()
        torch.cuda.synchronize()
        t_real = real["num_actual_tokens"]
        out, conv, ssm = st.g.host_out(), st.g.host_conv(), st.g.host_ssm()
        # the oracle on the unpadded batch
        ref_out, ref_conv, ref_ssm = helpers.run_case(real)
        assert_out_close(out[:t_real], ref_out)
        np.testing.assert_array_equal(conv, ref_conv)
        named = synth.referenced_slots(real)
        if len(named):
            assert_states_close(ssm[named], ref_ssm[named])
        rest = np.setdiff1d(np.arange(ssm.shape[0]), named)
        np.testing.assert_array_equal(ssm[rest], real["ssm_state"][rest])
        # and the eager call on the unpadded batch, bit for bit
        np.testing.assert_array_equal(out[:t_real], eager.host_out())
        np.testing.assert_array_equal(conv, eager.host_conv())
        np.testing.assert_array_equal(ssm, eager.host_ssm())


def test_graph_padded_spec_replays():
    # spec-only graph: the padded step uses the first NS_PAD * K input rows
    _run_graph(False, [(300, 8, 0), (301, 5, 0), (302, 2, 0), (303, 8, 0), (304, 1, 0)])


def test_graph_vhead_units_replays():
    # padded to 104 spec rows of four tokens and 32 v-heads plus the decodes:
    # a launch that carries both runs one workgroup per (row, k-head), with
    # the turn counters passed and left untouched, replay after replay
    _run_graph(True, [(350, 104, 6), (351, 40, 3), (352, 104, 0), (353, 0, 6), (354, 77, 5)],
               ns_pad=104, num_slots=500, k=4, heads=(16, 32))


def test_graph_vhead_tail_replays():
    # spec rows alone, padded to 104 rows of four tokens and 32 v-heads: the
    # captured step runs one workgroup per (row, v-head) and per CU, its last
    # units claimed at run time through the turn array's NULL-slot cell, so
    # every replay must find that count back at 0; the eager calls on the
    # real batches take the same form with a tail (104, 77 and 40 rows) or
    # several workgroups per CU and no tail (8 rows)
    _run_graph(False, [(360, 104, 0), (361, 40, 0), (362, 104, 0), (363, 8, 0), (364, 77, 0)],
               ns_pad=104, num_slots=500, k=4, heads=(16, 32))


def test_graph_padded_decodes_and_spec_replays():
    _run_graph(True, [(310, 8, 6), (311, 3, 4), (312, 6, 0), (313, 0, 5), (314, 8, 6)])


def test_graph_padded_prefills_replays():
    # decodes + prefill rows (chunked form, dk = 128) + spec rows in one
    # captured step; the real prefill rows change length replay by replay
    _run_graph(True, [(330, 8, 6, [130, 64]), (331, 3, 4, [65]), (332, 5, 0, []),
                      (333, 0, 2, [1, 199]), (334, 8, 6, [200])])


@pytest.mark.parametrize("seed", range(3))
def test_graph_random_replays(seed):
    # one captured step (decodes + prefills + spec rows at their padded
    # sizes) replayed over six seeded batches: any number of real spec rows
    # and decodes up to the pads (none included), up to two prefill rows
    # whose lengths fit the token budget
    rng = np.random.default_rng(340 + seed)
    plan = []
    for i in range(6):
        n_pf = int(rng.integers(0, NP_PAD))
        cuts = np.sort(rng.integers(0, PF_TOK + 1, size=n_pf))
        pf = [int(x) for x in np.diff(np.concatenate([[0], cuts])) if x > 0]
        plan.append((3400 + 10 * seed + i, int(rng.integers(0, NS_PAD + 1)),
                     int(rng.integers(0, ND_PAD + 1)), pf))
    say(f"random graph plan {seed}: {plan}")
    _run_graph(True, plan)
