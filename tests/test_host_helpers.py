"""Host builds of the small helpers the kernels share with the host code (CPU only)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_join_words_never_sign_extends_the_low_word(tmp_path):
    # Regression: a 64-bit base rebuilt from wave-uniform 32-bit copies must keep a low word
    # with bit 31 set in the low half only.
    src = tmp_path / "join.cpp"
    src.write_text(r'''
#include <cstdio>
#include "attn_internal.h"
int main() {
    const uint64_t addrs[] = {0x00007f1280001000ull, 0x00007f12ffffffffull, 0x0000000080000000ull,
                              0x00007fff00000010ull, 0x1ull};
    for (uint64_t a : addrs)
        if (attn::join_words((uint32_t)(a >> 32), (uint32_t)a) != a) { std::printf("bad %llx\n", (unsigned long long)a); return 1; }
    return 0;
}
''')
    exe = tmp_path / "join"
    subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
                    os.path.join(ROOT, "verify_attention_e4m3_amd", "csrc"), str(src), "-o", str(exe)], check=True)
    subprocess.run([str(exe)], check=True)


def test_split_policy_host_copy_matches_partitions(tmp_path):
    # partition_len / num_splits compiled for the host cover [0, L): cap partitions up to
    # 131072 tokens, partitions of at most part_max (or L / 64) past it, never over 64 splits
    src = tmp_path / "pol.cpp"
    src.write_text(r'''
#include <cstdio>
#include "attn_internal.h"
int main() {
    const int caps[] = {8, 16, 32, 64};
    for (int cap : caps)
        for (int L = 1; L <= 262144; L += 37) {
            attn::SplitPolicy p{cap, attn::kLongLen / cap, 512, 256};
            const int P = attn::partition_len(L, p), S = attn::num_splits(L, p);
            if (P % 256 || P < 512 || S > attn::kMaxSplits || (long)(S - 1) * P >= L || (long)S * P < L) return 1;
            if (L <= attn::kLongLen && S > cap) return 2;
            const int fewest = ((L + 63) / 64 + 255) / 256 * 256;
            if (L > attn::kLongLen && P > (p.part_max > fewest ? p.part_max : fewest)) return 3;
            if (P > 16384) return 4;
        }
    return 0;
}
''')
    exe = tmp_path / "pol"
    subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
                    os.path.join(ROOT, "verify_attention_e4m3_amd", "csrc"), str(src), "-o", str(exe)], check=True)
    subprocess.run([str(exe)], check=True)
