"""sa_attention_noalloc, the entry point that allocates nothing (its index
and partials live in the library's own per-GPU device array), against
sa_attention with a caller workspace: outputs bit-identical on two calls in a
row, the second on a smaller input, through the C ABI. The array keeps the
previous call's contents, so the second call also shows that nothing stale
leaks into a smaller problem."""
import numpy as np
import pytest
import torch

import block_sparse_paged_csr_amd as sa
import oracle
import workloads as W
from _gpu import dev_inputs, max_rel_err, run_attention

pytestmark = pytest.mark.gpu


def _noalloc(w, d, out, lse):
    return sa.sa_attention_noalloc(d["q"], d["k"], d["v"], d["sel"], d["bt"], d["cu"], d["used"],
                                   w.block_size, w.softmax_scale, w.causal, out, lse,
                                   check=False, return_index=True)


def test_noalloc_matches_sa_attention_twice():
    big = W.make_config("decode")
    small = W.make_random(4242, batch=3, qo_max=5, kv_max=200, hkv=2, qhead=4, head_dim=128,
                          page_size=16, pages_per_block=2, topk=4)
    cases = [("decode", big), ("small", small)]
    inputs = [dev_inputs(w) for _, w in cases]
    refs = [run_attention(w, d) for (_, w), d in zip(cases, inputs)]     # caller workspace
    torch.cuda.synchronize()
    for i, ((name, w), d, (ref_out, ref_lse)) in enumerate(zip(cases, inputs, refs)):
        print(f"[gpu case] no-alloc call {i}: {name} tq={w.tq}", flush=True)
        out = torch.full_like(ref_out, 3.0)
        lse = torch.full_like(ref_lse, 3.0)
        torch.cuda.synchronize()
        before = (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0])
        _, _, idx = _noalloc(w, d, out, lse)
        torch.cuda.synchronize()
        after = (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0])
        assert after[0] == before[0], "torch allocated during the call"
        if i == 0:
            # first call on this GPU: the runtime loads the array with the
            # library's code object (the set-up the header documents)
            assert before[1] - after[1] <= sa.SA_NOALLOC_SCRATCH_BYTES + (8 << 20), (before, after)
        else:
            assert after[1] >= before[1], (before, after)      # no device allocation
        info = sa.sa_index_status(idx)
        assert info["status"] == 0
        assert torch.equal(out, ref_out), f"{name}: out differs from sa_attention"
        assert torch.equal(lse, ref_lse), f"{name}: lse differs from sa_attention"
        ref_o, _ = oracle.attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected,
                                           w.block_tables, w.cu_seqlens_q, w.used_kv_lens, w.hq,
                                           w.hkv, w.head_dim, w.block_size, w.page_size,
                                           w.softmax_scale, w.causal)
        err, _ = max_rel_err(out.cpu().numpy(), ref_o)
        assert err <= 1e-4, f"{name}: O rel err {err:.3e}"


def test_noalloc_reports_device_errors():
    w = W.make_random(4343, batch=2, hkv=1, topk=2, head_dim=32)
    d = dev_inputs(w)
    sel = w.selected.copy()
    sel.reshape(-1)[0] = 10 ** 6
    d["sel"] = torch.from_numpy(sel).cuda()
    out = torch.zeros((w.tq, w.hq, w.head_dim), device="cuda")
    with pytest.raises(sa.SaError) as ei:
        sa.sa_attention_noalloc(d["q"], d["k"], d["v"], d["sel"], d["bt"], d["cu"], d["used"],
                                w.block_size, w.softmax_scale, w.causal, out, None, check=True)
    assert ei.value.kind == "SelectedOutOfRange"
    assert torch.all(torch.isnan(out))
