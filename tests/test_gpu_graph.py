"""hipGraph replay of the sequential and micro-batched baselines.

Every replay, with eager device work on the same stream between replays, must
equal the kernel-by-kernel run (CP_FLAG_EAGER) bit for bit; a new pointer set
is captured anew and old ones stay valid through the plan's bounded cache; a
run issued while the caller captures its own stream is recorded kernel by
kernel into the caller's graph and replays correctly."""
import sys

import pytest

from tile_dependency_pipelined_amd import inputs as gen

pytestmark = pytest.mark.gpu

M, WIDTHS, TILE, MB = 512, (512, 768, 512), (128, 128), 128


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    from tile_dependency_pipelined_amd import chain as ch
    from tile_dependency_pipelined_amd import native as nat
    assert torch.cuda.is_available()
    X, Ws = gen.chain_inputs(M, WIDTHS, gen.BF16, 1.0, [k ** -0.5 for k in WIDTHS[:-1]], 77)
    dX = ch.to_device(X, gen.BF16)
    dW = [ch.to_device(w, gen.BF16) for w in Ws]
    ref = {}
    with ch.Chain(M, list(WIDTHS), gen.BF16, *TILE, flags=nat.CP_FLAG_EAGER) as c:
        for mode in ("sequential", "microbatch"):
            dY = torch.empty((M, WIDTHS[-1]), dtype=torch.bfloat16, device="cuda")
            c.run(dX, dW, dY, mode=mode, microbatch_rows=MB if mode == "microbatch" else 0)
            assert c.stats()["status"] == 0
            ref[mode] = dY.clone()
    return {"torch": torch, "ch": ch, "nat": nat, "dX": dX, "dW": dW, "ref": ref}


def same(a, b):
    import torch
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("mode", ["sequential", "microbatch"])
def test_replays_match_eager(env, mode):
    torch, ch = env["torch"], env["ch"]
    say(f"graph replay {mode}: M={M} widths={WIDTHS} tile={TILE}")
    mb = MB if mode == "microbatch" else 0
    dY = torch.empty((M, WIDTHS[-1]), dtype=torch.bfloat16, device="cuda")
    scratch = torch.randn(256, 256, device="cuda")
    with ch.Chain(M, list(WIDTHS), gen.BF16, *TILE) as c:
        for rep in range(5):
            dY.fill_(float("nan"))                  # eager work between replays
            scratch = scratch @ scratch.t() / 256.0
            c.run(env["dX"], env["dW"], dY, mode=mode, microbatch_rows=mb)
            st = c.stats()
            assert st["status"] == 0, st
            torch.cuda.synchronize()
            assert same(dY, env["ref"][mode]), f"replay {rep} differs from the eager run"


def test_pointer_changes_and_cache_eviction(env):
    torch, ch = env["torch"], env["ch"]
    say("graph cache: 18 output buffers, both baseline modes")
    outs = [torch.empty((M, WIDTHS[-1]), dtype=torch.bfloat16, device="cuda") for _ in range(18)]
    with ch.Chain(M, list(WIDTHS), gen.BF16, *TILE) as c:
        for sweep in range(2):
            for k, y in enumerate(outs):
                mode = "sequential" if k % 2 == 0 else "microbatch"
                y.fill_(float("nan"))
                c.run(env["dX"], env["dW"], y, mode=mode, microbatch_rows=MB if mode == "microbatch" else 0)
                assert c.stats()["status"] == 0
                torch.cuda.synchronize()
                assert same(y, env["ref"][mode]), f"sweep {sweep} buffer {k} ({mode})"


@pytest.mark.parametrize("mode", ["sequential", "microbatch"])
def test_inside_caller_capture(env, mode):
    torch, ch = env["torch"], env["ch"]
    say(f"caller capture {mode}")
    mb = MB if mode == "microbatch" else 0
    dY = torch.empty((M, WIDTHS[-1]), dtype=torch.bfloat16, device="cuda")
    with ch.Chain(M, list(WIDTHS), gen.BF16, *TILE) as c:
        c.run(env["dX"], env["dW"], dY, mode=mode, microbatch_rows=mb)   # warm, outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c.run(env["dX"], env["dW"], dY, mode=mode, microbatch_rows=mb)
        torch.cuda.synchronize()
        for rep in range(3):
            dY.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert same(dY, env["ref"][mode]), f"caller-graph replay {rep}"
        del g


def test_pipelined_capture_refused(env):
    torch, ch, nat = env["torch"], env["ch"], env["nat"]
    say("caller capture pipelined: refused")
    dY = torch.empty((M, WIDTHS[-1]), dtype=torch.bfloat16, device="cuda")
    with ch.Chain(M, list(WIDTHS), gen.BF16, *TILE) as c:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            with pytest.raises(nat.CpError) as ei:
                c.run(env["dX"], env["dW"], dY, mode="pipelined")
        torch.cuda.synchronize()
        assert ei.value.code == nat.CP_ERR_UNSUPPORTED
        c.run(env["dX"], env["dW"], dY, mode="pipelined")   # still usable outside capture
        assert c.stats()["status"] == 0
        torch.cuda.synchronize()
        assert same(dY, env["ref"]["sequential"])
        del g
