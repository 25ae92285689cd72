"""Host-side pieces of bench.py: the kernel source hash that ties a committed counter
summary to the kernel code it was taken on (no GPU needed)."""
import bench


def test_code_only_drops_comments_and_blank_lines():
    text = "int a = 1;  // one\n/* two\n   lines */ int b = 2;\n\n   \nint c = 3;   \n"
    assert bench._code_only(text) == "int a = 1;\n int b = 2;\nint c = 3;"


def test_code_only_keeps_code_changes():
    assert bench._code_only("x = a + b; // sum") != bench._code_only("x = a - b; // sum")


def test_kernel_source_hash_per_dtype():
    hb, hf = bench.kernel_source_hash("bf16"), bench.kernel_source_hash("fp8")
    assert len(hb) == len(hf) == 16 and hb != hf
    assert hb == bench.kernel_source_hash("bf16")
