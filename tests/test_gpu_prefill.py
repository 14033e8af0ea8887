"""Chunked prefill attention on the GPU (pkv_prefill_attention) against the
FP64 oracle (orc_prefill_attention) over the GPU's own cache read back:
causal attention of each sequence's last q_len cached tokens, within max-abs
2e-3 and row max-rel 1e-2. Whole prompts, chunks at an offset, one-token
chunks, ragged tiles; INT8 and FP16 layers; G 1/2/4; head_dim 64/128;
block sizes 16/32/64; fp32/bf16/fp16 queries; one context piece and the
context cut into pieces merged by log-sum-exp."""
import numpy as np
import pytest

from oracle import oracle as orc
from paged_kv_cache_62_amd import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


def _prefill(case, qlens, q_dtype, piece_tokens=0, max_context_len=None, workspace=None):
    import torch
    sh = case.shape
    pool = H.make_gpu_pool(case)
    o = H.replay(case, pool)  # the cache, written through pkv_append_kv
    torch.cuda.synchronize()
    seqs = case.decode_seqs
    maxb = max((int(pool.length(s)) + sh.bs - 1) // sh.bs for s in seqs)
    st, table, lens = o.alloc.table(seqs, maxb)
    assert st == orc.OK
    H.compare_caches(case, o, pool, seqs, maxb)  # bit-exact with the oracle's
    qstart = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    x = synth.normal(synth.stream_seed(case.seed, 4747), int(qstart[-1]) * sh.hq * sh.dim)
    q = synth.round_to(x.reshape(int(qstart[-1]), sh.hq, sh.dim), q_dtype)
    dev = pool.arena.device
    outs, refs = [], []
    rows = H.used_blocks_with_rows(o, seqs, table.shape[1])
    mctx = int(max(lens)) if max_context_len is None else max_context_len
    print(f"prefill case seed={case.seed} qlens={list(qlens)} piece_tokens={piece_tokens} max_ctx={mctx}",
          flush=True)
    for layer in range(sh.layers):
        out = pool.prefill(layer, q.to(dev), torch.from_numpy(qstart).to(dev), int(max(qlens)),
                           torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev), sh.scale, mctx,
                           workspace=workspace, piece_tokens=piece_tokens)
        torch.cuda.synchronize()
        kc, vc, ks, vs = H.gpu_layer_arrays(pool, layer, rows.keys(), sh)
        refs.append(orc.prefill_attention(sh.dtype(layer), kc, vc, ks, vs, synth.as_f32(q), qstart, table, lens,
                                          sh.scale))
        outs.append(out.cpu().numpy())
    got, ref = np.stack(outs), np.stack(refs)
    ma, mr = H.attention_errors(got, ref)
    return got, ref, ma, mr


def _case(kv, hq, hkv, dim, bs, lens, seed, in_dtype="bf16", sigma="per_head"):
    nblocks = sum((n + bs - 1) // bs for n in lens) + 6
    sh = H.Shape(layers=2, hq=hq, hkv=hkv, dim=dim, bs=bs, nblocks=nblocks, kv_dtype=kv, in_dtype=in_dtype,
                 q_dtype=in_dtype, free_order_seed=11, sigma_kv=sigma, outlier_p=0.01)
    return H.Case(sh, seed, [("allocate", s, n) for s, n in enumerate(lens)], decode_seqs=list(range(len(lens))))


@pytest.mark.parametrize("kv", [orc.I8, orc.F16])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (8, 2)])
@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("piece_tokens", [0, 64])
def test_prefill_whole_prompts_and_chunks(gpu, kv, hq, hkv, bs, piece_tokens):
    lens = [1, 15, 16, 47, 200, 333]
    qlens = [1, 15, 16, 47, 37, 100]      # whole prompts, then chunks at an offset
    c = _case(kv, hq, hkv, 128, bs, lens, 64000 + hq * 10 + bs + kv)
    got, ref, ma, mr = _prefill(c, qlens, "bf16", piece_tokens)
    print(f"prefill kv={kv} hq={hq} bs={bs} pieces of {piece_tokens}: max_abs={ma:.3e} max_rel={mr:.3e}",
          flush=True)
    H.assert_attention_close(got, ref)


@pytest.mark.parametrize("kv", [orc.I8, orc.F16])
@pytest.mark.parametrize("q_dtype", ["f32", "f16"])
@pytest.mark.parametrize("piece_tokens", [0, 128])
def test_prefill_head_dim_64_and_query_types(gpu, kv, q_dtype, piece_tokens):
    lens = [5, 64, 130]
    c = _case(kv, 4, 2, 64, 32, lens, 64100 + kv, in_dtype=q_dtype, sigma="unit")
    got, ref, ma, mr = _prefill(c, [5, 33, 130], q_dtype, piece_tokens)
    print(f"prefill d64 kv={kv} q={q_dtype}: max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
    H.assert_attention_close(got, ref)


def test_prefill_one_token_chunks_equal_decode(gpu):
    """A chunk of one query is a decode step: the prefill kernel and the
    decode kernel agree within the tolerance on the same cache."""
    import torch
    c = _case(orc.I8, 8, 2, 128, 16, [1, 77, 500], 64200)
    res = H.run_decode_case(c, partition_tokens=0)
    pool = res["pool"]
    dev = pool.arena.device
    q = res["q"].to(dev)
    qstart = torch.arange(4, dtype=torch.int32, device=dev)
    for layer in range(c.shape.layers):
        out = pool.prefill(layer, q, qstart, 1, torch.from_numpy(res["table"]).to(dev),
                           torch.from_numpy(res["lens"]).to(dev), c.shape.scale, int(res["lens"].max()))
        H.assert_attention_close(out.cpu().numpy(), res["ref"][layer])


@pytest.mark.parametrize("kv", [orc.I8, orc.F16])
@pytest.mark.parametrize("piece_tokens", [0, 192])
def test_prefill_many_tiles(gpu, kv, piece_tokens):
    """Many tiles (4 sequences x 8 KV heads, chunks of 530-600 queries with
    G = 2), the context whole or in pieces of 192 tokens: several pieces per
    workgroup of queries, the last partial."""
    lens = [600, 620, 545, 700]
    c = _case(kv, 16, 8, 128, 16, lens, 64300 + kv)
    got, ref, ma, mr = _prefill(c, [600, 530, 545, 580], "bf16", piece_tokens)
    print(f"prefill many tiles kv={kv}: max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
    H.assert_attention_close(got, ref)
    # P's hi + lo parts carry ~22 bits, so the error sits near 2e-5 here; a
    # hi part rounded twice (once for the product, once for the lo
    # subtraction) showed up as ~2.5e-3 on this case
    assert ma < 2e-4, f"max abs error {ma:.3e}: P split lost precision"


def test_prefill_context_longer_than_planned(gpu):
    """max_context_len below the real contexts (only max_query_len is
    checked against it): the pieces are planned from it and the last piece
    takes the rest of each context, so the result is still whole."""
    lens = [300, 455, 210]
    c = _case(orc.I8, 8, 2, 128, 16, lens, 64400)
    got, ref, ma, mr = _prefill(c, [40, 64, 17], "bf16", piece_tokens=64, max_context_len=128)
    print(f"prefill short plan: max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
    H.assert_attention_close(got, ref)


def test_prefill_plan_and_workspace_checks(gpu):
    """The plan reports the split and its workspace; a launch that needs a
    workspace rejects a missing or short one on the host."""
    import torch
    from paged_kv_cache_62_amd import pkv
    c = _case(orc.I8, 8, 2, 128, 16, [300, 455], 64500)
    pool = H.make_gpu_pool(c)
    T, n, nb = pool.prefill_plan(pkv.PKV_BF16, 8, 2, 64, 455, 64)
    assert (T, n) == (64, 8) and nb == pkv.MERGE_COUNTER_BYTES + 2 * 64 * 8 * n * (2 + 128) * 4
    assert pool.prefill_plan(pkv.PKV_BF16, 8, 2, 64, 455, 0)[1:] == (1, 0)  # short contexts: one piece
    dev = pool.arena.device
    q = torch.zeros(128, 8, 128, dtype=torch.bfloat16, device=dev)
    qs = torch.tensor([0, 64, 128], dtype=torch.int32, device=dev)
    table = torch.zeros(2, 29, dtype=torch.int32, device=dev)
    lens = torch.tensor([300, 455], dtype=torch.int32, device=dev)
    short = torch.empty(nb - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(pkv.PkvError):
        pool.prefill(0, q, qs, 64, table, lens, 1.0, 455, workspace=short, piece_tokens=64)
    with pytest.raises(pkv.PkvError):
        pool.prefill(0, q, qs, 64, table, lens, 1.0, 455, piece_tokens=96)  # not a multiple of 64
    with pytest.raises(pkv.PkvError):
        pool.prefill(0, q, qs, 64, table, lens, 1.0, 32)  # max_context_len < max_query_len


def test_prefill_workspace_reused(gpu):
    """One workspace for every call: the pieces' arrival counters are back at
    zero after each launch, so later launches of other shapes (both layers,
    then shorter chunks with fewer tile groups) merge correctly in it."""
    import torch
    from paged_kv_cache_62_amd import pkv
    lens = [600, 620, 545, 700]
    c = _case(orc.I8, 16, 8, 128, 16, lens, 64500)
    sh = c.shape
    big = [600, 530, 545, 580]
    pool = H.make_gpu_pool(c)
    _, _, nb = pool.prefill_plan(pkv.PKV_BF16, sh.hq, len(lens), max(big), max(lens), 192)
    slots = len(lens) * max(big) * sh.hq * -(-max(lens) // 192)
    assert nb == pkv.MERGE_COUNTER_BYTES + slots * (2 + sh.dim) * 4
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for qlens in (big, [70, 1, 200, 33], big):
        got, ref, ma, mr = _prefill(c, qlens, "bf16", piece_tokens=192, max_context_len=max(lens), workspace=ws)
        print(f"prefill reused workspace qlens={qlens}: max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
        H.assert_attention_close(got, ref)
        assert int(torch.count_nonzero(ws[:pkv.MERGE_COUNTER_BYTES])) == 0, "arrival counters not left at zero"


@pytest.mark.parametrize("kv,hq,hkv,dim,bs,q_dtype,lens,qlens,piece_tokens", [
    (orc.I8, 16, 8, 128, 16, "bf16", [2100, 2600], [128, 100], 0),
    (orc.I8, 16, 8, 128, 16, "bf16", [2100, 2600], [128, 100], 512),
    (orc.F16, 8, 2, 64, 32, "f32", [2200, 3000], [64, 40], 0),
    (orc.I8, 4, 4, 128, 64, "f16", [2500, 2048], [256, 200], 0),
    (orc.F16, 16, 8, 128, 16, "bf16", [2300, 2050], [128, 70], 0),
])
def test_prefill_eight_wavefronts(gpu, kv, hq, hkv, dim, bs, q_dtype, lens, qlens, piece_tokens):
    """Few query tiles over long contexts: the automatic plan cuts the
    context, and the launch runs eight wavefronts per workgroup (twice the
    tiles per staged step; some of them past the chunk), merged over ragged
    piece counts. INT8 and FP16, head_dim 64 and 128, G 1/2/4, fp32, fp16
    and bf16 queries, automatic and explicit pieces."""
    from paged_kv_cache_62_amd import pkv
    c = _case(kv, hq, hkv, dim, bs, lens, 64600 + hq + dim + bs + kv, in_dtype=q_dtype)
    pool = H.make_gpu_pool(c)
    qcode = {"f32": pkv.PKV_F32, "f16": pkv.PKV_F16, "bf16": pkv.PKV_BF16}[q_dtype]
    T, n, _, waves = pool.prefill_plan(qcode, hq, len(lens), max(qlens), max(lens), piece_tokens, waves=True)
    assert waves == 8 and n > 1, (T, n, waves)
    got, ref, ma, mr = _prefill(c, qlens, q_dtype, piece_tokens)
    print(f"prefill eight wavefronts kv={kv} hq={hq}/{hkv} d={dim} q={q_dtype} pieces {n} x {T}: "
          f"max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
    H.assert_attention_close(got, ref)


def test_prefill_workspace_shared_by_four_and_eight_wavefront_launches(gpu):
    """One workspace for launches whose arrival counters are laid out
    differently (an eight-wavefront launch over long contexts, then a
    four-wavefront launch cut into explicit pieces, then the first again):
    each leaves the counter prefix at zero and matches the oracle."""
    import torch
    from paged_kv_cache_62_amd import pkv
    long_case = _case(orc.I8, 16, 8, 128, 16, [2100, 2600], 64700)
    short_case = _case(orc.I8, 16, 8, 128, 16, [600, 620, 545, 700], 64701)
    pool = H.make_gpu_pool(long_case)
    assert pool.prefill_plan(pkv.PKV_BF16, 16, 2, 128, 2600, 0, waves=True)[3] == 8
    assert pool.prefill_plan(pkv.PKV_BF16, 16, 4, 600, 700, 192, waves=True)[3] == 4
    nb = max(pool.prefill_plan(pkv.PKV_BF16, 16, 2, 128, 2600, 0)[2],
             pool.prefill_plan(pkv.PKV_BF16, 16, 4, 600, 700, 192)[2])
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for case, qlens, T in ((long_case, [128, 100], 0), (short_case, [600, 530, 545, 580], 192),
                           (long_case, [128, 100], 0)):
        got, ref, ma, mr = _prefill(case, qlens, "bf16", piece_tokens=T, workspace=ws)
        print(f"prefill shared workspace qlens={qlens} pieces of {T}: max_abs={ma:.3e} max_rel={mr:.3e}",
              flush=True)
        H.assert_attention_close(got, ref)
        assert int(torch.count_nonzero(ws[:pkv.MERGE_COUNTER_BYTES])) == 0, "arrival counters not left at zero"


@pytest.mark.parametrize("ragged", [False, True])
def test_prefill_eight_wavefronts_over_rounds(gpu, ragged):
    """Whole prompts whose four-wavefront grid would take two rounds: the
    plan runs eight wavefronts per workgroup with one piece (G = 4 so that
    eight 512-token prompts reach that size; ragged lengths leave some
    workgroups' second half past the chunk)."""
    from paged_kv_cache_62_amd import pkv
    lens = [512 - (37 * i) % 200 if ragged else 512 for i in range(8)]
    c = _case(orc.I8, 32, 8, 64, 16, lens, 64800 + int(ragged))
    pool = H.make_gpu_pool(c)
    plan = pool.prefill_plan(pkv.PKV_BF16, 32, 8, max(lens), max(lens), 0, waves=True)
    assert plan[1] == 1 and plan[3] == 8, plan
    got, ref, ma, mr = _prefill(c, lens, "bf16")
    print(f"prefill eight wavefronts over rounds ragged={ragged}: max_abs={ma:.3e} max_rel={mr:.3e}", flush=True)
    H.assert_attention_close(got, ref)
