"""The training-loop robustness calls on the GPU: the optimizer step split
into gpt2_grad_norm + gpt2_adamw_update (bit-identical to
gpt2_clip_and_adamw), the guarded step that skips an update whose gradient
norm spikes (llm.c GPT-2 1.5B post, dszhyy.com, 400B-token run section: skip on a
loss or norm z-score above 5), and checkpoint / resume reproducing the
uninterrupted run bit for bit (same post, flags section)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import transformer_lm_pretraining_train_amd as g  # noqa: E402
from gpu_util import host, to_dev  # noqa: E402

LR = 1e-3


def case(dtype="fp32", k=2, name="tiny"):
    wl = synth.workload(name).replace(grad_accum=k)
    cfg = g.config_for(wl, dtype)
    layout = [(n, o, s) for n, o, s, _ in g.param_layout(cfg)]
    flat = synth.init_params(layout, wl.n_layer, wl.vocab_size, [wl.seed_id, 2])
    stream = synth.token_stream(wl, wl.micro_batch * wl.seq_len * k * 6 + 1)
    batches = [synth.micro_batch(stream, i, wl.micro_batch, wl.seq_len) for i in range(6 * k)]
    dev = [(to_dev(x), to_dev(y)) for x, y in batches]
    return cfg, flat, dev, k


def grads_of(m, dev, step, k):
    m.zero_grad()
    loss = torch.zeros(1, device="cuda")
    for x, y in dev[step * k:(step + 1) * k]:
        m.forward(x, y, loss)
        m.backward()
    return float(loss)


def state(m):
    mm, vv, t = m.get_opt_state()
    torch.cuda.synchronize()
    return host(m.get_params()), host(mm), host(vv), t


def new_model(cfg, flat):
    m = g.Model(cfg)
    m.set_params(to_dev(flat))
    return m


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_two_call_step_matches_clip_and_adamw(dtype):
    cfg, flat, dev, k = case(dtype)
    a, b = new_model(cfg, flat), new_model(cfg, flat)
    for step in range(2):
        grads_of(a, dev, step, k)
        a.clip_and_adamw(LR)
        grads_of(b, dev, step, k)
        with pytest.raises(g.GPT2Error) as ei:  # no norm since the backward
            b.adamw_update(LR)
        assert ei.value.name == "ESTATE"
        norm = b.grad_norm(1.0)
        assert np.isfinite(norm) and norm > 0
        b.adamw_update(LR)
        with pytest.raises(g.GPT2Error):  # the norm is used up
            b.adamw_update(LR)
    for x, y in zip(state(a), state(b)):
        assert np.array_equal(x, y)


def test_guarded_step_skips_a_gradient_spike_and_a_nonfinite_norm():
    cfg, flat, dev, k = case("fp32")
    m = new_model(cfg, flat)
    lz, nz = g.ZScore(4), g.ZScore(4)
    applied = 0
    for step in range(5):  # history; thresholds off so that every step applies
        loss = grads_of(m, dev, step, k)
        r = m.guarded_step(loss, LR, lz, nz, z_max_loss=0.0, z_max_norm=0.0)
        assert not r["skipped"]
        applied += 1
        if step < 4:
            assert np.isnan(r["z_norm"])
    before = state(m)
    assert before[3] == applied
    loss = grads_of(m, dev, 5, k)
    m.set_grads(m.get_grads() * 1000.0)  # a spike in the gradient norm
    r = m.guarded_step(loss, LR, lz, nz, z_max_loss=5.0, z_max_norm=5.0)
    assert r["skipped"] and r["z_norm"] > 5.0
    after = state(m)
    for x, y in zip(before, after):
        assert np.array_equal(x, y)
    assert m.skip_counts() == {"nonfinite": 0, "outlier": 1}
    gv = m.get_grads()
    gv[7] = float("nan")
    m.set_grads(gv)
    with pytest.raises(g.GPT2Error) as ei:
        m.guarded_step(loss, LR, lz, nz)
    assert ei.value.name == "ENONFINITE"
    for x, y in zip(before, state(m)):
        assert np.array_equal(x, y)
    assert m.skip_counts() == {"nonfinite": 1, "outlier": 1}


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_resume_from_checkpoint_is_bitwise(dtype, tmp_path):
    cfg, flat, dev, k = case(dtype)
    a = new_model(cfg, flat)
    for step in range(2):
        grads_of(a, dev, step, k)
        a.clip_and_adamw(LR)
    gv = a.get_grads()
    gv[0] = float("nan")
    a.set_grads(gv)
    with pytest.raises(g.GPT2Error):  # a skip, so the counts are non-trivial
        a.clip_and_adamw(LR)
    path = tmp_path / "state.ckpt"
    a.save_state(str(path))
    for step in range(2, 4):
        grads_of(a, dev, step, k)
        a.clip_and_adamw(LR)
    b = g.Model(cfg)  # fresh: parameters, m, v, step all zero
    b.load_state(str(path))
    assert b.skip_counts() == {"nonfinite": 1, "outlier": 0}
    for step in range(2, 4):
        grads_of(b, dev, step, k)
        b.clip_and_adamw(LR)
    sa, sb = state(a), state(b)
    assert sa[3] == sb[3] == 4
    for x, y in zip(sa[:3], sb[:3]):
        assert np.array_equal(x, y)


def test_guarded_run_resumes_bitwise_with_its_detector_windows(tmp_path):
    """A guarded run (gpt2_guarded_step with loss and norm detectors whose
    windows are full) checkpointed between steps, the detectors' windows
    saved beside the file, resumes on a fresh model and fresh detectors and
    matches the uninterrupted run bit for bit: parameters, m, v, step, skip
    counts and every z-score."""
    cfg, flat, dev, k = case("bf16")
    win = 3

    def run(m, lz, nz, steps):
        out = []
        for step in steps:
            grads_of(m, dev, step, k)
            r = m.guarded_step(10.0 + 0.01 * step, LR, loss_z=lz, norm_z=nz)
            out.append((r["z_loss"], r["z_norm"], r["skipped"]))
        return out

    a = new_model(cfg, flat)
    la, na = g.ZScore(win), g.ZScore(win)
    run(a, la, na, range(3))  # windows full
    path = tmp_path / "guarded.ckpt"
    a.save_state(str(path))
    saved = (la.get_state(), na.get_state())
    assert len(saved[0]) == win and len(saved[1]) == win
    za = run(a, la, na, range(3, 6))
    b = g.Model(cfg)
    b.load_state(str(path))
    lb, nb = g.ZScore(win), g.ZScore(win)
    lb.set_state(saved[0])
    nb.set_state(saved[1])
    zb = run(b, lb, nb, range(3, 6))
    for x, y in zip(za, zb):
        assert np.array_equal(np.array(x, dtype=np.float64), np.array(y, dtype=np.float64))
    assert all(np.isfinite(z[1]) for z in za)  # the norm windows were full: real z-scores
    sa, sb = state(a), state(b)
    assert sa[3] == sb[3]
    for x, y in zip(sa[:3], sb[:3]):
        assert np.array_equal(x, y)
    assert a.skip_counts() == b.skip_counts()


def test_checkpoint_rejects_other_shapes_and_bad_files(tmp_path):
    cfg, flat, dev, k = case("fp32")
    a = new_model(cfg, flat)
    path = tmp_path / "a.ckpt"
    a.save_state(str(path))
    other = synth.workload("tiny").replace(n_layer=synth.workload("tiny").n_layer + 1)
    b = g.Model(g.config_for(other, "fp32"))
    with pytest.raises(g.GPT2Error) as ei:
        b.load_state(str(path))
    assert ei.value.name == "EINVAL"
    data = path.read_bytes()
    short = tmp_path / "short.ckpt"
    short.write_bytes(data[:len(data) - 4])
    c = g.Model(cfg)
    with pytest.raises(g.GPT2Error):
        c.load_state(str(short))
    bad = tmp_path / "bad.ckpt"
    bad.write_bytes(b"NOTACKPT" + data[8:])
    with pytest.raises(g.GPT2Error):
        c.load_state(str(bad))
    with pytest.raises(g.GPT2Error):
        c.load_state(str(tmp_path / "missing.ckpt"))
    # the loaded state equals the saved one
    c.load_state(str(path))
    for x, y in zip(state(a), state(c)):
        assert np.array_equal(x, y)
