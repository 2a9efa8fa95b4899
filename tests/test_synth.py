"""The seeded input recipe stays what the design notes state: split sizes of every
workload, their structure (empty groups, ranges), and checksums of the 8-group
workload's first x block and first weight group.  A change to the generator that
would silently change every measured and tested input fails here."""
import numpy as np

import synth

W8 = synth.WORKLOADS["bf16_train_g8_k4096_n14336"]


def test_eight_group_splits_and_input_checksums():
    m = synth.split_sizes(W8)
    assert m.tolist() == [2033, 2039, 2055, 2130, 2024, 2073, 1983, 2047]
    assert synth.checksum(m) == "5124f9588d44c481"
    # block i of x comes from child i alone, so the first block of any T >= 1024 is the same
    assert synth.checksum(synth.x(W8.scaled(T=1024))) == "86c679b6add93d8f"
    assert synth.checksum(synth.weight_group(W8, 0)) == "fd8db1ca938a6279"


def test_other_workloads_split_structure():
    z = synth.split_sizes(synth.WORKLOADS["bf16_zipf_g64_k2048_n1536"])
    assert z.sum() == 65536 and (z == 0).sum() == 4 and z.max() == 19929
    assert synth.checksum(z) == "16264b52646f29b1"
    g256 = synth.split_sizes(synth.WORKLOADS["bf16_fwd_g256_k7168_n2048_outbuf"])
    assert g256.sum() == 32768 and g256.min() == 103 and g256.max() == 157
    mx = synth.split_sizes(synth.WORKLOADS["mxfp8_fwd_g32_k4096_n4096"])
    assert mx.sum() == 32768 and mx.min() == 985 and mx.max() == 1087
    assert synth.split_sizes(synth.WORKLOADS["fwd_f32_g4_k64_n32"]).tolist() == [5, 0, 17, 10]


def test_checksum_is_of_the_raw_bytes():
    a = np.arange(6, dtype=np.int64)
    assert synth.checksum(a) == synth.checksum(a.reshape(2, 3))
    assert synth.checksum(a) != synth.checksum(a[::-1])
