"""Full-model parity: 32 stacked 8B-shape layers (seeds 4000..4031, context
32768 per layer, 16 KV splits: the launch configuration bench.py times for
the full-model step), the final norm, the bf16 LM head 128256 x 4096 and the
greedy argmax, against the CPU oracle, for 16 seeded input rows.

Every row runs through the library exactly as the full-model step does (32
one-launch block steps at M = 1, then i4d_lm_head_argmax).  The checks:

* teacher-forced per layer: oracle layer l consumes the GPU's output of
  layer l-1 for the same 16 rows (so 32 layers of bf16 rounding do not
  compound against one fixed bound); block output rel-RMS <= 1e-2 and
  attention max-abs/RMS <= 2e-2 at every layer;
* the token appended by the last row's step at every layer is bit-exact
  against the oracle's encoding of the step's own bf16 key and value;
* LM head, teacher-forced on the GPU's final hidden rows: logits rel-RMS
  <= 1e-4, and the GPU's token equals the oracle's argmax for every row,
  except where the oracle's top-1 / top-2 gap is below the measured logit
  error (a near-tie);
* end to end, one row through the oracle's own 32 layers (no teacher
  forcing): reported, beside the oracle's own chain run again on the same
  row with one bf16 ulp added to 1% of its input entries.  Layers with
  N(0, 0.02^2) random weights amplify a difference by about 1.3x per
  layer (the perturbed oracle chain diverges from the unperturbed one like
  the GPU's does), so after 32 layers neither end-to-end comparison is
  near the per-layer bound and neither is asserted.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
from int4_quantized_decode_amd import synth
from tests.gpu_helpers import assert_appended_exact, bf16_values, norm_maxabs, rel_rms, say
from tests.test_gpu_stages import gpu  # noqa: F401

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROWS = 16
REL_TOL = 1e-2
ATT_TOL = 2e-2


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 4
    return max(2, min(12, n))


def _row_caches(base: O.RowCache, n: int):
    return [O.RowCache(base.k_codes.copy(), base.k_scales.copy(), base.v_codes.copy(), base.v_scales.copy())
            for _ in range(n)]


def _near_tie_ok(gpu_tok, ref_logits, logit_err):
    """The GPU's token is the oracle's argmax, or the two differ by less
    than the measured logit error in the oracle's own logits."""
    ref_tok = int(np.argmax(ref_logits))
    if gpu_tok == ref_tok:
        return True, 0.0
    gap = float(ref_logits[ref_tok] - ref_logits[gpu_tok])
    return gap <= logit_err, gap


def test_full_model_32_layers_lm_head_argmax(gpu):
    torch, B, D = gpu
    wl = synth.WORKLOADS["8b_32layer_ctx32768"]
    shape, L, nl, S = wl.shape, wl.ctx, wl.n_layers, wl.num_splits
    assert (L, nl, S) == (32768, 32, 16)
    seeds = [wl.seed + l for l in range(nl)]
    lengths = np.array([L], np.int32)
    workers = _workers()
    t0 = time.time()

    # the oracle's encodings of each layer, taken from the same host arrays
    # the library's packer reads (the two encoders share no code)
    def encode(seed, lw, pre):
        ql = O.quantize_layer(lw)
        base = O.build_cache(shape, [L], pre)[0]
        return ql, base

    say(f"c4: building {nl} layers with {workers} host threads")
    layers, caches, enc = D.stacked_layers(shape, seeds, lengths, workers=workers, on_host=encode)
    V, d = synth.LM_VOCAB, shape.d_model
    w_lm, g_lm = synth.make_lm_head(d, V, synth.LM_HEAD_SEED)
    w16 = D.to_device_u16(B.i4d_pack_lm_head(w_lm, g_lm))
    say(f"c4: set-up {time.time() - t0:.0f} s")

    ws = D.Workspace(shape, 1, L, S)
    lm_bytes = B.i4d_lm_head_workspace_bytes(V, 1)
    lm_ws = torch.zeros(lm_bytes, dtype=torch.uint8, device="cuda")
    ctx = torch.from_numpy(lengths).cuda()
    x_rows = synth.make_x(shape, ROWS, wl.seed)              # [16, d] bf16 bits
    hd, nkv = shape.head_dim, shape.n_kv_heads
    outs = np.zeros((nl, ROWS, d), np.uint16)                # GPU block outputs (bf16 bits)
    attns = np.zeros((nl, ROWS, shape.n_q_heads * hd), np.float32)
    logits = np.zeros((ROWS, V), np.float32)
    toks = np.zeros(ROWS, np.int64)
    bufs = [torch.empty((1, d), dtype=torch.int16, device="cuda") for _ in range(2)]
    attn = torch.empty((1, shape.n_q_heads * hd), dtype=torch.float32, device="cuda")
    lg = torch.empty((1, V), dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    for i in range(ROWS):
        cur = D.to_device_u16(x_rows[i:i + 1])
        for l in range(nl):
            out = bufs[l % 2]
            B.i4d_decode_block_step(layers[l].struct, caches[l].struct, cur, out, ctx, 1, L, S, ws.buf, ws.nbytes,
                                    attn)
            if i == ROWS - 1:
                torch.cuda.synchronize()
                assert_appended_exact(caches[l], ws, shape, lengths)
            outs[l, i] = D.to_host_u16(out)[0]
            attns[l, i] = attn.cpu().numpy()[0]
            cur = out
        B.i4d_lm_head_argmax(w16, V, d, cur, 1, shape.rms_eps, lg, tok, lm_ws, lm_bytes)
        torch.cuda.synchronize()
        logits[i] = lg.cpu().numpy()[0]
        toks[i] = int(tok.item())
    for c in caches:
        assert c.errors() == 0
    say(f"c4: GPU passes done at {time.time() - t0:.0f} s; tokens {toks.tolist()}")

    # teacher-forced oracle, one layer per task
    def tf_layer(l):
        ql, base = enc[l]
        x_in = x_rows if l == 0 else outs[l - 1]
        ref = O.decode_block(shape, ql, _row_caches(base, ROWS), x_in, [L] * ROWS)
        e_out = rel_rms(synth.bf16_bits_to_f32(outs[l]), ref.out)
        e_att = norm_maxabs(attns[l], ref.attn)
        return e_out, e_att

    # one row end to end through the oracle's own layers (sequential), and
    # the same chain on a perturbed copy of the row
    def free_running(x):
        hidden = []
        for l in range(nl):
            ql, base = enc[l]
            ref = O.decode_block(shape, ql, _row_caches(base, 1), x, [L])
            hidden.append(ref.out[0])
            x = synth.f32_to_bf16_bits(ref.out.astype(np.float32))
        return np.array(hidden)

    x_pert = x_rows[:1].copy()
    idx = np.random.default_rng(1).choice(d, d // 100, replace=False)
    x_pert[0, idx] += 1   # one bf16 ulp (bit pattern + 1) at 1 % of the entries

    with ThreadPoolExecutor(workers) as ex:
        fr = ex.submit(free_running, x_rows[:1])
        frp = ex.submit(free_running, x_pert)
        tf = list(ex.map(tf_layer, range(nl)))
        fr_hidden, frp_hidden = fr.result(), frp.result()
    for l, (e_out, e_att) in enumerate(tf):
        say(f"  layer {l:2d}: out rel-RMS {e_out:.3e}  attn max-abs/rms {e_att:.3e}")
    say(f"c4: oracle layers done at {time.time() - t0:.0f} s")
    assert max(e for e, _ in tf) <= REL_TOL
    assert max(a for _, a in tf) <= ATT_TOL

    # LM head on the GPU's final hidden rows (teacher-forced)
    w_hat = O.lm_head_weight_bf16(w_lm, g_lm)
    del w_lm
    h_gpu = bf16_values(outs[nl - 1])
    ref_logits, ref_tok = O.lm_head_argmax(h_gpu, w_hat, shape.rms_eps)
    e_lm = rel_rms(logits, ref_logits)
    logit_err = float(np.abs(logits - ref_logits).max())
    say(f"c4: LM head logits rel-RMS {e_lm:.3e}, max |error| {logit_err:.3e}; oracle tokens {ref_tok.tolist()}")
    assert e_lm <= 1e-4
    agree = 0
    for i in range(ROWS):
        ok, gap = _near_tie_ok(int(toks[i]), ref_logits[i], logit_err)
        agree += int(toks[i]) == int(ref_tok[i])
        assert ok, (i, int(toks[i]), int(ref_tok[i]), gap, logit_err)
        assert int(toks[i]) == int(np.argmax(logits[i]))  # the GPU's argmax of its own logits
    say(f"c4: argmax agreement {agree}/{ROWS} (the rest near-ties)")

    # end to end (row 0): the oracle's own chain (reported)
    e_gpu = [rel_rms(synth.bf16_bits_to_f32(outs[l, 0]), fr_hidden[l]) for l in range(nl)]
    e_pert = [rel_rms(frp_hidden[l], fr_hidden[l]) for l in range(nl)]
    fr_logits, fr_tok = O.lm_head_argmax(fr_hidden[nl - 1:], w_hat, shape.rms_eps)
    for l in (0, 1, 3, 7, 15, 23, 31):
        say(f"  end to end, layer {l:2d}: GPU vs oracle chain {e_gpu[l]:.3e}; oracle chain vs the oracle chain on "
            f"a 1-ulp perturbed input {e_pert[l]:.3e}")
    say(f"c4: end-to-end token row 0: gpu {int(toks[0])} oracle chain {int(fr_tok[0])}; total {time.time() - t0:.0f} s")
    # the first layer's end-to-end difference is the per-layer one
    assert e_gpu[0] <= REL_TOL
