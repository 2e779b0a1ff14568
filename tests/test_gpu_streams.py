"""Calls on several HIP streams at once (GPU).

The library keeps no state between calls: every launch takes its inputs,
outputs and workspace from the caller, so independent calls on different
streams may overlap on the device.  Each case runs a few steps on the default
stream for reference outputs, then the same steps concurrently on two streams
(of the default priority) and requires the same bits."""
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, log

pytestmark = pytest.mark.gpu


def _decode_case(lens, seed):
    seqs = [W.SeqSpec("decode", int(L), 1) for L in lens]
    return W.build(f"streams-dec-{seed}", seed, "bf16", 32, 8, 128, 16, seqs)


def _prefill_case(pairs, seed):
    seqs = [W.SeqSpec("prefill", int(lk), int(lq)) for lq, lk in pairs]
    return W.build(f"streams-pre-{seed}", seed, "bf16", 32, 8, 128, 64, seqs)


def _outputs(steps):
    return [s.dec_out.clone() if s.dec else s.pre_out.clone() for s in steps]


@pytest.mark.parametrize("planned", [False, True], ids=["one-launch", "planned"])
def test_concurrent_streams_match_sequential_bitwise(planned):
    steps = [DeviceStep(_decode_case([3000, 17, 900, 4100, 256], seed=31)),
             DeviceStep(_prefill_case([(300, 1200), (64, 64), (513, 2000)], seed=32)),
             DeviceStep(_decode_case([128, 5000, 2048], seed=33))]

    def run(s):
        s.store()
        if s.pre:
            s.prefill(planned)
        if s.dec:
            s.decode()

    for s in steps:
        run(s)
    torch.cuda.synchronize()
    ref = _outputs(steps)
    streams = [torch.cuda.Stream() for _ in range(2)]
    for rep in range(3):
        log(f"concurrent streams, repeat {rep}, planned={planned}")
        for s in steps:  # fresh outputs, so that a skipped write cannot pass
            (s.dec_out if s.dec else s.pre_out).fill_(float("nan"))
        torch.cuda.synchronize()
        for i, s in enumerate(steps):
            with torch.cuda.stream(streams[i % 2]):
                run(s)
        torch.cuda.synchronize()
        for got, want in zip(_outputs(steps), ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))
