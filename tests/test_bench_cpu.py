"""Host logic of bench.py: the source hash that keys the measured traffic
ignores comments and blank lines but not code, and every measured-traffic key
names a workload, a tile height and a hash of the right form."""
import bench


def _hash_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.source_hash((str(p),))


def test_source_hash_ignores_comments_and_blank_lines(tmp_path):
    code = "int f(int a)\n{\n    return a + 1;\n}\n"
    commented = ("// a comment\nint f(int a) // trailing\n{\n\n    /* block\n       comment */\n    return a + 1;   \n}\n")
    assert _hash_of(tmp_path, code) == _hash_of(tmp_path, commented)


def test_source_hash_follows_code(tmp_path):
    assert _hash_of(tmp_path, "int f(int a) { return a + 1; }\n") != _hash_of(tmp_path, "int f(int a) { return a + 2; }\n")


def test_source_sets_cover_the_roofline_kernels():
    assert "paged_expert_weight_amd/csrc/moe_gemm.hip" in bench.GEMM_SOURCES
    assert "paged_expert_weight_amd/csrc/decode.hip" in bench.DECODE_SOURCES
    assert "paged_expert_weight_amd/csrc/route_token.h" in bench.DECODE_SOURCES
    assert len(bench.gemm_source_hash()) == len(bench.decode_source_hash()) == 16


def test_measured_traffic_keys():
    for (name, T, bm, atomic, h), v in bench.MEASURED_TRAFFIC.items():
        assert name in ("tiny", "qwen15", "decode", "mixtral", "qwen3n")
        assert T > 0 and bm in (16, 32, 64, 128, 256) and atomic in (False, True)
        assert len(h) == 16 and int(h, 16) >= 0
        assert v > 0
