// zc_table_emit.cpp -- build step: runs the table generator and writes the
// constants of table_id 1 as initializer macros for the kernels.
#include <cstdio>

#include "zc_table.h"

static void row(const char* name, const unsigned* v, int n)
{
    std::printf("#define %s {", name);
    for (int i = 0; i < n; ++i)
        std::printf("%s%u", i ? "," : "", v[i]);
    std::printf("}\n");
}

int main()
{
    zc::Table t;
    if (!zc::build_table(&t)) {
        std::fprintf(stderr, "zc_table_emit: table generation failed\n");
        return 1;
    }
    unsigned buf[1 << zc::kLutBits];
    std::printf("// Generated at build time by zc_table_emit (zc_table.cpp).\n");
    std::printf("#define ZC_T1_NSYM %d\n", zc::kSymbols);
    int maxlen = 0;
    for (int s = 0; s < zc::kSymbols; ++s) {
        buf[s] = static_cast<unsigned>(t.len[s]);
        if (t.len[s] > maxlen)
            maxlen = t.len[s];
    }
    row("ZC_T1_LEN_INIT", buf, zc::kSymbols);
    std::printf("#define ZC_T1_MAXLEN %d\n", maxlen);
    for (int s = 0; s < zc::kSymbols; ++s)
        buf[s] = t.code[s];
    row("ZC_T1_CODE_INIT", buf, zc::kSymbols);
    for (int i = 0; i < (1 << zc::kLutBits); ++i)
        buf[i] = t.lut[i];
    std::printf("#define ZC_T1_LUT_BITS %d\n", zc::kLutBits);
    std::printf("#define ZC_T1_TAIL_BITS %d\n", zc::kTailBits);
    row("ZC_T1_LUT_INIT", buf, 1 << zc::kLutBits);
    for (int L = 0; L <= zc::kMaxCodeLen; ++L)
        buf[L] = t.limit[L];
    row("ZC_T1_LIMIT_INIT", buf, zc::kMaxCodeLen + 1);
    for (int L = 0; L <= zc::kMaxCodeLen; ++L)
        buf[L] = static_cast<unsigned>(t.base[L]);
    row("ZC_T1_BASE_INIT", buf, zc::kMaxCodeLen + 1);
    for (int r = 0; r < zc::kSymbols; ++r)
        buf[r] = t.sorted_sym[r];
    row("ZC_T1_SORTED_INIT", buf, zc::kSymbols);
    std::printf("#define ZC_T1_TAIL_OK %d\n", t.tail_ok ? 1 : 0);
    for (int i = 0; i < (1 << zc::kTailBits); ++i)
        buf[i] = t.tail[i];
    row("ZC_T1_TAIL_INIT", buf, 1 << zc::kTailBits);
    std::printf("#define ZC_T1_ESC_LEN %d\n", t.len[zc::kEscape]);
    return 0;
}
