/* Exhaustive round trip of the oracle's INT4 word packing over all 2^32
 * words: pack(unpack(w)) == w, and every unpacked code lies in [-8, 7].
 * Test helper: links the oracle library, prints "mismatches=<n> ...".
 * The word range is split over OpenMP threads; each word is independent. */
#include <stdint.h>
#include <stdio.h>

uint32_t orc_pack_word(const int8_t q[8]);
void orc_unpack_word(uint32_t w, int8_t q[8]);

int main(void)
{
    unsigned long long bad = 0, out_of_range = 0;
#pragma omp parallel for reduction(+ : bad, out_of_range) schedule(static)
    for (long long hi = 0; hi < 65536; ++hi) {
        int8_t q[8];
        for (uint32_t lo = 0; lo < 65536; ++lo) {
            uint32_t w = ((uint32_t)hi << 16) | lo;
            orc_unpack_word(w, q);
            for (int k = 0; k < 8; ++k)
                out_of_range += (q[k] < -8 || q[k] > 7);
            bad += orc_pack_word(q) != w;
        }
    }
    printf("mismatches=%llu out_of_range=%llu\n", bad, out_of_range);
    return bad || out_of_range;
}
