// Host-side check of the compact fragment layout of the per-chunk T and P
// matrices (gdn_chunk.hpp: tri_frag_off, tri_frag_at, tri_frag_half), the
// layout that prep_kernel writes to the workspace and the chain kernels read
// back. Both matrices are lower triangular (T unit lower, P including its
// diagonal), so the layout must (1) store every entry on or below the
// diagonal exactly once, (2) drop only entries above it, and (3) tile its
// kTriFragBytes bytes exactly, 8 bytes per stored half-lane. Exit status 0
// when all hold; the first violation is printed.
#include <cstdio>
#include <vector>

#include "gdn_chunk.hpp"

int main() {
    using namespace gdn;
    constexpr int N = 64;
    std::vector<int> cover(N * N, 0);
    std::vector<int> bytes(kTriFragBytes, 0);
    for (int i = 0; i < kTriFrags; ++i) {
        const int rb = tri_rb(i), k2 = tri_k2(i);
        if (tri_frag(rb, k2) != i) {
            printf("fragment %d: tri_frag(tri_rb, tri_k2) = %d\n", i, tri_frag(rb, k2));
            return 1;
        }
        for (int l = 0; l < 64; ++l) {
            const int g4 = l >> 4, c16 = l & 15, row = 16 * rb + c16;
            for (int h = 0; h < 2; ++h) {
                const bool stored = !(tri_frag_half(i) && h == 1);
                for (int e = 0; e < 4; ++e) {
                    const int col = 32 * k2 + 4 * g4 + 16 * h + e;
                    if (stored) {
                        cover[row * N + col] += 1;
                    } else if (col <= row) {
                        printf("fragment %d lane %d half %d drops entry (%d, %d) on or below the diagonal\n",
                               i, l, h, row, col);
                        return 1;
                    }
                }
                if (!stored) continue;
                const int off = tri_frag_at(i, l, h);
                if (off < 0 || off + 8 > kTriFragBytes || off % 8 != 0) {
                    printf("fragment %d lane %d half %d: offset %d outside the %d bytes\n", i, l, h, off,
                           kTriFragBytes);
                    return 1;
                }
                for (int b = 0; b < 8; ++b) bytes[off + b] += 1;
            }
        }
    }
    for (int r = 0; r < N; ++r)
        for (int c = 0; c <= r; ++c)
            if (cover[r * N + c] != 1) {
                printf("entry (%d, %d) stored %d times\n", r, c, cover[r * N + c]);
                return 1;
            }
    for (int b = 0; b < kTriFragBytes; ++b)
        if (bytes[b] != 1) {
            printf("byte %d written %d times\n", b, bytes[b]);
            return 1;
        }
    printf("compact fragment layout ok: %d bytes per matrix\n", kTriFragBytes);
    return 0;
}
