"""Failure containment on the GPU: a NaN in one sample's inputs stays in that
sample.  Every step of the target is per sample (the shared timestep, the
per-sample key counts, the per-(sample, modality) norms of deep read section
3.1, E6), so the other samples' J, gbar, norms and loss must come out bit for
bit as in a clean run.  NaN data cannot fault the GPU; the check is that no
reduction, split-tail merge or batched GEMM mixes samples."""
import numpy as np
import pytest

from joint_video_audio_trigflow_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CFG = inputs.Config("nan-containment", B=3, Nv=300, Na=45, Nt=20, Ntv=13, Cv=128, Ca=64, d=256, H=2,
                    in_dtype="bf16", beta=1.5, gamma=0.7, mask_mode="scatter", index=41)


def run(problem, dmd=False):
    from joint_video_audio_trigflow_amd import _lib
    cfg = problem["cfg"]
    if dmd:
        dev = _lib.to_device_dmd_problem(problem)
        out = _lib.DmdTarget(cfg)(dev["teacher"], dev["fake"], dev["x0_v"], dev["x0_a"], dev["eps_v"],
                                  dev["eps_a"], dev["text"], dev["text_mask"], dev["t"])
    else:
        dev = _lib.to_device_problem(problem)
        out = _lib.ScmTarget(cfg)(dev["teacher"], dev["student"], dev["z0_v"], dev["z0_a"], dev["eps_v"],
                                  dev["eps_a"], dev["text"], dev["text_mask"], dev["t"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


@pytest.mark.parametrize("precision", ["bf16", "split"])
@pytest.mark.parametrize("where", ["z0_v", "z0_a", "text"])
def test_nan_in_one_sample_stays_there(where, precision):
    print(f"NaN containment: {where} of sample 1 ({precision})", flush=True)
    cfg = CFG.replace(precision=precision)
    p = inputs.make_problem(cfg)
    clean = run(p)
    data = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
    if where == "text":
        valid = np.flatnonzero(data["text_mask"][1])
        data["text"][1, valid[0], 5] = np.nan   # a valid text key of sample 1
    else:
        data[where][1, 7, 3] = np.nan
    bad = run(dict(p, data=data))
    for k in clean:
        assert np.array_equal(clean[k][[0, 2]], bad[k][[0, 2]]), k   # other samples: bit for bit
    assert not np.isfinite(bad["loss"][1])                            # the NaN is not hidden either


def test_nan_in_one_sample_stays_there_dmd():
    print("NaN containment: DMD term, x0_v of sample 1", flush=True)
    p = inputs.make_dmd_problem(CFG)
    clean = run(p, dmd=True)
    data = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p["data"].items()}
    data["x0_v"][1, 11, 2] = np.nan
    bad = run(dict(p, data=data), dmd=True)
    for k in clean:
        assert np.array_equal(clean[k][[0, 2]], bad[k][[0, 2]]), k
    assert not np.isfinite(bad["loss"][1])
