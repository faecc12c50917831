"""The benchmark's byte accounting, derived again from the shapes the pages
print (tests/golden/page_facts.json): the headline rate divides these bytes
by the step time, so a wrong count would misstate every figure.

Algorithmic bytes count what the method must move once: K and V of every
visible key (bf16, 2 bytes), the queries read and the outputs written, and
for the fused calls the new tokens read and stored.  Split-K partials and
the padded tail are overhead, not algorithmic bytes.
"""
import json
import os

import bench

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
BF16 = 2


def test_bench_workload_matches_the_pages():
    assert bench.B == FACTS["decode_batch"]["value"]
    assert bench.W == FACTS["sliding_window"]["window"]
    assert (bench.HKV, bench.D) == (FACTS["attention_shapes"]["sliding"]["kv_heads"],
                                    FACTS["attention_shapes"]["sliding"]["head_dim"])
    assert (bench.GHKV, bench.GD) == (FACTS["attention_shapes"]["global"]["kv_heads"],
                                      FACTS["attention_shapes"]["global"]["head_dim"])
    assert bench.GG * bench.GS == FACTS["grouped_verify_rows"]["rows"]
    assert bench.KC == FACTS["global_key_count"]["value"]


def test_algorithmic_bytes_of_the_step():
    decode, append_s, glob, append_g = bench.algorithmic_bytes()
    # sliding decode: every request's full window of K and V per KV head
    # (positions >= W, so the window is full), one query row per q head in,
    # one out
    q_heads = bench.HKV * bench.G
    kv = bench.B * bench.W * bench.HKV * bench.D * BF16 * 2
    assert kv == 469_762_048
    assert decode == kv + 2 * bench.B * q_heads * bench.D * BF16 == 473_432_064
    # its append: one token's K and V per request and KV head, read and stored
    assert append_s == bench.B * bench.HKV * bench.D * BF16 * 2 * 2 == 917_504
    # global verify: the 6005 keys (not the 6016 padded), 32 rows in and out
    kv_g = bench.KC * bench.GHKV * bench.GD * BF16 * 2
    assert kv_g == 24_596_480
    rows = bench.GHKV * bench.GG * bench.GS
    assert glob == kv_g + 2 * rows * bench.GD * BF16 == 24_727_552
    assert append_g == bench.GS * bench.GHKV * bench.GD * BF16 * 2 * 2 == 32_768
    # the padded tail the kernels may touch is not counted
    padded = FACTS["global_key_count"]["padded_to"]
    assert (padded - bench.KC) * bench.GHKV * bench.GD * BF16 * 2 == 45_056


def test_traffic_is_tied_to_the_kernel_code_not_its_comments(tmp_path):
    """The roofline's counter traffic is reported only while the kernel
    sources hash to the value recorded with the counters: a comment or blank
    line edit keeps the hash, any code edit changes it."""
    src = ("// kernel\n__global__ void k(float* x) {\n  /* two\n     lines */ x[0] = 1.f;  // store\n\n}\n")
    variants = {
        "same": src,
        "comment": src.replace("// store", "// the store").replace("/* two", "/* three"),
        "blank": src.replace("\n\n", "\n\n\n"),
        "code": src.replace("1.f", "2.f"),
        "code_in_comment_line": src.replace("// kernel\n", "// kernel\nint z;\n"),
    }
    hashes = {}
    for name, text in variants.items():
        f = tmp_path / f"{name}.hip"
        f.write_text(text)
        hashes[name] = bench.kernel_source_hash([str(f)])
    assert hashes["comment"] == hashes["same"] == hashes["blank"]
    assert hashes["code"] != hashes["same"]
    assert hashes["code_in_comment_line"] != hashes["same"]
